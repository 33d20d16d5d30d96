"""Pins of the verify-acceptance oracle (thinkspread, 'The economics of
speculative decoding': greedy acceptance, rollback, rolling gate and the
break-even acceptance of the cost model)."""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle.verify import (RollingGate, argmax_rows, break_even_acceptance, expected_tokens,
                           greedy_accept, rollback_len)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_hand.json")


def test_hand_worked_example():
    g = json.load(open(GOLDEN))
    logits = np.array(g["logits"], dtype=np.float32)
    assert argmax_rows(logits).tolist() == g["argmax"]
    for st in g["steps"]:
        acc, nxt, _ = greedy_accept(logits, np.array(st["draft"]))
        assert (acc, nxt) == (st["accepted"], st["next"])
        assert rollback_len(g["P"], acc) == st["rollback"]


def _argmax_brute(row):
    """First index of the largest value; a NaN beats every number."""
    best = 0
    for j in range(1, len(row)):
        a, b = row[j], row[best]
        if math.isnan(b):
            continue
        if math.isnan(a) or a > b:
            best = j
    return best


@pytest.mark.parametrize("seed", range(6))
def test_argmax_matches_brute_force_with_ties_and_nans(seed):
    g = np.random.default_rng(seed)
    x = g.integers(-3, 4, size=(7, 40)).astype(np.float32)  # many ties
    if seed % 2:
        x[g.integers(0, 7, 3), g.integers(0, 40, 3)] = np.nan
    x[0, :] = -0.0
    x[0, 5] = 0.0  # -0.0 == +0.0: the first one wins
    want = [_argmax_brute(r.tolist()) for r in x]
    assert argmax_rows(x).tolist() == want


@pytest.mark.parametrize("n_match", [0, 1, 2, 3])
def test_planted_drafts_are_accepted_up_to_the_first_mismatch(n_match):
    logits, drafts, planted = synth.verify_case(5, 4, 1000, n_match)
    acc, nxt, t = greedy_accept(logits, drafts)
    assert t.tolist() == planted[:, 0].tolist()
    assert acc == n_match
    assert nxt == planted[acc, 0]


def test_tie_goes_to_lowest_id():
    logits, drafts, planted = synth.verify_case(6, 3, 500, 0, tie=True)
    assert argmax_rows(logits).tolist() == planted.min(axis=1).tolist()


def test_expected_tokens_closed_forms():
    for k in range(0, 7):
        assert expected_tokens(1.0, k) == k + 1
        assert expected_tokens(0.0, k) == 1
        a = 0.37
        assert expected_tokens(a, k) == pytest.approx((1 - a ** (k + 1)) / (1 - a), rel=1e-12)


def test_break_even_closed_forms():
    a, b = 9.0, 5.5  # the page's cost model, verify(m) = 9 + 5.5 m (ms)
    # k = 1: (1 + alpha)(a + b) = a + 2b
    assert break_even_acceptance(a, b, 1) == pytest.approx(b / (a + b), abs=1e-12)
    # k = 2: alpha^2 + alpha + 1 = (a + 3b) / (a + b)
    need = (a + 3 * b) / (a + b)
    assert break_even_acceptance(a, b, 2) == pytest.approx((-1 + math.sqrt(4 * need - 3)) / 2,
                                                           abs=1e-12)
    assert break_even_acceptance(a, b, 0) == 0.0
    assert break_even_acceptance(1.0, 1e6, 1) == pytest.approx(1e6 / (1e6 + 1), abs=1e-9)


def test_page_gate_threshold_matches_the_page_cost_model_at_k3():
    """Two printed numbers of the page tie together through the cost model:
    with verify(m) = 9 + 5.5 m and the default depth k = 3, speculation breaks
    even at a per-position acceptance of about 0.59, next to the 0.60 gate."""
    alpha = break_even_acceptance(9.0, 5.5, 3)
    assert expected_tokens(alpha, 3) * 14.5 == pytest.approx(9.0 + 5.5 * 4, abs=1e-9)
    assert abs(alpha - 0.60) < 0.02


def test_gate_keeps_high_acceptance_and_closes_on_low():
    g = RollingGate(3, 0.60, window=4)
    for _ in range(20):  # 0.92-like: 3 of 3 and 2 of 3 alternating (mean 0.83)
        assert g.step(3) == 3
        assert g.step(2) == 3
    g = RollingGate(3, 0.60, window=4)
    ks = [g.step(a) for a in (3, 3, 0, 0, 1, 3, 3)]
    # rolling means: 1, 1, 2/3, 1/2 -> closed at the fourth step, for good
    assert ks == [3, 3, 3, 0, 0, 0, 0]


def test_gate_window_forgets_old_steps():
    g = RollingGate(2, 0.60, window=2)
    assert [g.step(a) for a in (0, 2, 2)] == [0, 0, 0]  # first step: 0.0 < 0.6
    g = RollingGate(2, 0.60, window=2)
    assert [g.step(a) for a in (2, 1, 1, 2)] == [2, 2, 0, 0]  # (0.5 + 0.5) / 2 < 0.6
    g = RollingGate(2, 0.50, window=2)
    assert [g.step(a) for a in (2, 0, 2, 1)] == [2, 2, 2, 2]  # means 1, .5, .5, .75
    assert RollingGate(0).step(0) == 0
