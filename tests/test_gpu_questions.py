"""GPU parity of several questions about one resident state (openjev-
multimodal, "Latency", section "What changed": prefix priming) against the
oracle: each question sees the prefix and its own rows, nothing is
appended, and the result equals separate extends of the prefix."""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle.attention import extend_attention_questions
from tests.gpu_helpers import (announce, dev_bf16, env, host_bits, host_f64_of_bf16,
                               require_gpu)

pytestmark = pytest.mark.gpu
ATTN_TOL = 1e-2  # max-abs against the fp64 oracle


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _state(hq, hkv, d, prefix, ms, seed, cap=None):
    total = int(sum(ms))
    c = synth.attention_case(seed, hq, hkv, d, prefix, total)
    st = sve.KVSlots(1, 1, hq, hkv, d, cap or (prefix + total + 64), max(prefix, total, 1))
    slot, reused = st.kv_slot_select(np.arange(prefix + 1, dtype=np.int32))
    assert (slot, reused) == (0, 0)
    if prefix:
        st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                       dev_bf16(c["v_prefix"]))
    return c, st


QCASES = [
    # hq, hkv, d, prefix, question rows
    (32, 8, 128, 1250, [30, 24, 36, 27]),    # 4B-like state, four short questions
    (28, 4, 128, 1668, [254]),               # one question = an ordinary extend
    (28, 4, 128, 700, [1, 2, 3, 64, 65]),    # ragged, tiny and tile-sized questions
    (8, 2, 128, 0, [20, 45]),                # no prefix
    (8, 2, 128, 63, [5] * 16),               # sixteen questions
    (4, 2, 64, 130, [7, 70]),                # head_dim 64
    (32, 8, 128, 2048, [3, 2]),              # verify-sized questions on a long state
]


@pytest.mark.parametrize("case", QCASES, ids=lambda c: "h%d-%d-d%d-P%d-q%d" % (c[:4] + (len(c[4]),)))
def test_questions_match_oracle_and_leave_the_state(case):
    hq, hkv, d, prefix, ms = case
    announce(f"questions {case}")
    c, st = _state(hq, hkv, d, prefix, ms, seed=50 + len(ms))
    before = [host_bits(t) for t in st.kv_read(0, 0, 0, prefix)] if prefix else None
    out = st.extend_attn_questions(0, 0, ms, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]))
    want = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], ms)
    assert np.abs(host_f64_of_bf16(out) - want).max() <= ATTN_TOL
    assert st.kv_len(0, 0) == prefix  # nothing appended
    if prefix:
        after = [host_bits(t) for t in st.kv_read(0, 0, 0, prefix)]
        assert all(np.array_equal(a, b) for a, b in zip(before, after))


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_questions_under_forced_splits(splits):
    hq, hkv, d, prefix, ms = 28, 4, 128, 900, [40, 33, 50]
    announce(f"questions splits={splits}")
    c, st = _state(hq, hkv, d, prefix, ms, seed=61)
    with env(SVE_KV_SPLIT=splits):
        out = st.extend_attn_questions(0, 0, ms, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                       dev_bf16(c["v"]))
    want = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], ms)
    assert np.abs(host_f64_of_bf16(out) - want).max() <= ATTN_TOL


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["uniform", "cached-new", "balanced"])
@pytest.mark.parametrize("case", [(28, 4, 128, 1668, [100, 90, 64]), (8, 2, 128, 0, [200, 150]),
                                  (4, 2, 64, 500, [33, 1, 96])],
                         ids=lambda c: "h%d-%d-d%d-P%d-q%d" % (c[:4] + (len(c[4]),)))
def test_questions_under_each_split_layout(case, layout):
    """Questions whose bands cross the split boundaries of every table
    filling (a question's rows and keys spread over several pieces)."""
    hq, hkv, d, prefix, ms = case
    announce(f"questions layout={layout} {case}")
    c, st = _state(hq, hkv, d, prefix, ms, seed=71)
    with env(SVE_ATTN_LAYOUT=layout):
        out = st.extend_attn_questions(0, 0, ms, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                       dev_bf16(c["v"]))
    want = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], ms)
    assert np.abs(host_f64_of_bf16(out) - want).max() <= ATTN_TOL
    assert st.kv_len(0, 0) == prefix


def test_questions_equal_separate_extends():
    """One call with four questions against four extends of the prefix, each
    cut back to the prefix afterwards (the previous way: the prefix is read
    four times). Same rows within the tolerance."""
    hq, hkv, d, prefix, ms = 32, 8, 128, 800, [30, 24, 36, 27]
    announce("questions vs separate extends")
    total = int(sum(ms))
    c, st = _state(hq, hkv, d, prefix, ms, seed=62)
    st.kv_slot_select(np.arange(prefix + max(ms), dtype=np.int32))  # same slot, reuse P
    assert st.kv_len(0, 0) == prefix
    out = host_f64_of_bf16(st.extend_attn_questions(0, 0, ms, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                                    dev_bf16(c["v"])))
    r = 0
    for m in ms:
        sep = st.extend_attn(0, 0, dev_bf16(c["q"][r:r + m]), dev_bf16(c["k"][r:r + m]),
                             dev_bf16(c["v"][r:r + m]))
        st.kv_truncate(0, prefix)
        assert np.abs(host_f64_of_bf16(sep) - out[r:r + m]).max() <= ATTN_TOL
        r += m
    assert r == total


def test_questions_bad_arguments():
    c, st = _state(8, 2, 128, 64, [4], seed=63)
    q, k, v = dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"])
    with pytest.raises(sve.SveError):
        st.extend_attn_questions(0, 0, [4, 0], torch.zeros((4, 8, 128), dtype=torch.bfloat16,
                                                            device="cuda"), k, v)
    with pytest.raises(sve.SveError):
        st.extend_attn_questions(3, 0, [4], q, k, v)
    big = [1] * 17
    with pytest.raises(sve.SveError):
        st.extend_attn_questions(0, 0, big, torch.zeros((17, 8, 128), dtype=torch.bfloat16,
                                                        device="cuda"),
                                 torch.zeros((17, 2, 128), dtype=torch.bfloat16, device="cuda"),
                                 torch.zeros((17, 2, 128), dtype=torch.bfloat16, device="cuda"))
