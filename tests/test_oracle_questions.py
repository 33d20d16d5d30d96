"""Pins of the several-questions oracle (openjev-multimodal, "Latency",
section "What changed": prefix priming, each question resuming from the
shared prefix and reading only its own text). CPU only."""
import math

import numpy as np
import pytest

import synth
from oracle.attention import (_bf16_to_f64, extend_attention, extend_attention_questions)


def _questions(seed, hq, hkv, d, prefix, ms):
    c = synth.attention_case(seed, hq, hkv, d, prefix, int(sum(ms)))
    return c


def _masked_bruteforce(c, prefix, ms):
    """Attention over every key of the call (prefix + all questions' rows)
    with an explicit mask: row i of question j sees prefix keys and the rows
    of question j up to itself. Loops and math.fsum; tiny shapes only."""
    q = _bf16_to_f64(c["q"])
    k = _bf16_to_f64(np.concatenate([c["k_prefix"], c["k"]]))
    v = _bf16_to_f64(np.concatenate([c["v_prefix"], c["v"]]))
    m, hq, d = q.shape
    g = hq // k.shape[1]
    starts = np.concatenate([[0], np.cumsum(ms)[:-1]])
    out = np.zeros((m, hq, d))
    for j, (s0, mj) in enumerate(zip(starts, ms)):
        for i in range(s0, s0 + mj):
            keys = list(range(prefix)) + list(range(prefix + s0, prefix + i + 1))
            for h in range(hq):
                kv = h // g
                sc = [math.fsum(q[i, h, e] * k[t, kv, e] for e in range(d)) / math.sqrt(d)
                      for t in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                den = math.fsum(w)
                for e in range(d):
                    out[i, h, e] = math.fsum(w[a] * v[t, kv, e] for a, t in enumerate(keys)) / den
    return out


@pytest.mark.parametrize("prefix,ms", [(0, [2, 3]), (4, [1, 1, 1]), (5, [3, 2, 4]), (3, [1, 5])])
def test_matches_masked_bruteforce(prefix, ms):
    c = _questions(7, 4, 2, 8, prefix, ms)
    got = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], ms)
    assert np.abs(got - _masked_bruteforce(c, prefix, ms)).max() <= 1e-12


def test_one_question_is_an_extend():
    c = _questions(8, 8, 2, 16, 30, [12])
    got = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], [12])
    want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                            np.concatenate([c["v_prefix"], c["v"]]), 30)
    assert np.array_equal(got, want)


def test_questions_do_not_see_each_other():
    """Changing question 2's rows leaves question 1's outputs unchanged, and
    swapping the questions swaps the outputs."""
    ms = [5, 7]
    c = _questions(9, 8, 4, 16, 20, ms)
    base = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], ms)
    k2, v2 = c["k"].copy(), c["v"].copy()
    k2[5:] = synth.normal_bf16(synth.rng(1), k2[5:].shape)
    v2[5:] = synth.normal_bf16(synth.rng(2), v2[5:].shape)
    other = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], k2, v2, ms)
    assert np.array_equal(base[:5], other[:5])
    assert not np.allclose(base[5:], other[5:])
    perm = np.concatenate([np.arange(5, 12), np.arange(0, 5)])
    swapped = extend_attention_questions(c["q"][perm], c["k_prefix"], c["v_prefix"], c["k"][perm],
                                         c["v"][perm], [7, 5])
    assert np.array_equal(swapped, base[perm])


def test_pins_catch_questions_seeing_earlier_questions():
    """A plausible mistake (question rows also seeing the earlier questions'
    rows, i.e. one causal extend of everything) fails the brute-force pin."""
    ms = [3, 3]
    c = _questions(10, 4, 2, 8, 4, ms)
    wrong = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                             np.concatenate([c["v_prefix"], c["v"]]), 4)
    assert np.abs(wrong - _masked_bruteforce(c, 4, ms)).max() > 1e-3
