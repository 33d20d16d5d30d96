"""The library's prompt-lookup drafting (a host function behind the C ABI)
against the oracle: hand-worked cases, random histories with small
vocabularies (many repeats), long histories, and argument checks."""
import ctypes as C
import json
import os

import numpy as np
import pytest

import speculative_verify_extend_amd as sve
from speculative_verify_extend_amd import _lib
from oracle.ngram import ngram_draft

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_hand.json")


def test_hand_worked_cases():
    for c in json.load(open(GOLDEN))["cases"]:
        got = sve.ngram_draft(c["tokens"], c["k"], c["max_ngram"], c["min_ngram"]).tolist()
        assert got == c["draft"], c["why"]


@pytest.mark.parametrize("seed", range(200))
def test_random_histories_match_oracle(seed):
    g = np.random.default_rng(1000 + seed)
    n = int(g.integers(0, 300))
    tokens = g.integers(0, int(g.integers(2, 12)), n).astype(np.int32)
    k = int(g.integers(0, 9))
    lo = int(g.integers(1, 5))
    hi = lo + int(g.integers(0, 4))
    assert sve.ngram_draft(tokens, k, hi, lo).tolist() == ngram_draft(tokens.tolist(), k, hi, lo)


def test_long_history_with_planted_repeat():
    g = np.random.default_rng(7)
    t = g.integers(1000, 150000, 4000).astype(np.int32)  # essentially no repeats
    t[-3:] = t[1200:1203]  # the suffix planted at 1200
    got = sve.ngram_draft(t, 8, 3, 2)
    assert got.tolist() == t[1203:1211].tolist() == ngram_draft(t.tolist(), 8, 3, 2)


def test_argument_checks():
    lib = _lib.load()
    n = C.c_int32(0)
    buf = (C.c_int32 * 8)()
    toks = (C.c_int32 * 4)(1, 2, 1, 2)
    assert lib.sve_ngram_draft(toks, 4, -1, 3, 1, buf, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_ngram_draft(toks, 4, 65, 3, 1, buf, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_ngram_draft(toks, 4, 2, 1, 2, buf, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_ngram_draft(toks, 4, 2, 3, 0, buf, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_ngram_draft(None, 4, 2, 3, 1, buf, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_ngram_draft(toks, 4, 2, 3, 1, None, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_ngram_draft(toks, 4, 2, 3, 1, buf, C.byref(n)) == 0
    assert n.value == 2 and list(buf)[:2] == [1, 2]
