"""Pins of the slot-store / slot-selection oracle: exhaustive small cases,
the equivalent unique-argmax form, and the behaviours the goinfer page
reports ('Turn nine in under half a second', sections 'How it works',
'What was measured', 'What we got wrong')."""
import itertools

import numpy as np
import pytest

import synth
from oracle.slots import SlotOracle, lcp, unique_argmax_rule


def _fill(o, s, n):
    for layer in range(o.n_layers):
        o.extend(s, layer, n - o.kv_len[s][layer])


def _serve(o, prompt):
    """select + prefill the remainder in every layer; returns (slot, reused)."""
    s, r = o.select(prompt)
    _fill(o, s, len(prompt))
    return s, r


def test_lcp_basic():
    assert lcp([1, 2, 3], [1, 2, 4]) == 2
    assert lcp([], [1]) == 0
    assert lcp([5, 6], [5, 6, 7]) == 2


def _all_seqs(alphabet, max_len):
    for n in range(1, max_len + 1):
        yield from itertools.product(alphabet, repeat=n)


def test_exhaustive_small_cases():
    """All slot contents and prompts of length <= 3 over {0,1} with 3 slots:
    at most one eligible slot (asserted inside select), the literal rule is
    the unique-argmax rule, reuse never exceeds n-1, and the reused rows are
    exactly a common prefix of the stored tokens and the prompt."""
    seqs = [np.array(s) for s in _all_seqs((0, 1), 3)]
    choices = [None] + seqs
    count = 0
    for a, b, c in itertools.product(choices, repeat=3):
        for p in seqs:
            for literal in (False, True):
                o = SlotOracle(3, literal_rule=literal)
                for s, t in enumerate((a, b, c)):
                    if t is not None:
                        o.tokens[s] = t.copy()
                        o.kv_len[s] = [len(t)]
                        o.committed[s] = len(t)
                before = [o.resident(s).copy() for s in range(3)]
                el = o.eligible(p)
                if literal:
                    ua = unique_argmax_rule(p, [x if len(x) else None for x in before])
                    assert (el[0] if el else None) == ua
                s, r = o.select(p)
                assert 0 <= r <= len(p) - 1
                assert np.array_equal(before[s][:r], p[:r])
                count += 1
    assert count > 10000


def test_sampled_four_slot_cases():
    """20,000 random states of four slots whose contents have length 0..5
    over {0,1,2} (a third of them sharing a random common start), each with
    a random prompt of length 1..5: the same properties as the exhaustive
    test, for both rules."""
    g = np.random.default_rng(11)
    for i in range(20000):
        base = g.integers(0, 3, size=5)
        slots = []
        for _ in range(4):
            n = int(g.integers(0, 6))
            t = g.integers(0, 3, size=n)
            if i % 3 == 0 and n:
                k = int(g.integers(0, n + 1))
                t[:k] = base[:k]
            slots.append(t)
        p = g.integers(0, 3, size=int(g.integers(1, 6)))
        literal = bool(i & 1)
        o = SlotOracle(4, literal_rule=literal)
        for s, t in enumerate(slots):
            if len(t):
                o.tokens[s] = t.copy()
                o.kv_len[s] = [len(t)]
                o.committed[s] = len(t)
        before = [o.resident(s).copy() for s in range(4)]
        el = o.eligible(p)
        assert len(el) <= 1
        if literal:
            ua = unique_argmax_rule(p, [x if len(x) else None for x in before])
            assert (el[0] if el else None) == ua
        s, r = o.select(p)
        assert 0 <= r <= len(p) - 1
        assert np.array_equal(before[s][:r], p[:r])


def test_reuse_off_never_reuses():
    o = SlotOracle(4, reuse=False)
    for _, p in synth.rotation_sessions(1, 2, 4, 50, 7, 5, 9):
        s, r = _serve(o, p)
        assert r == 0


def test_repeated_prompt_reuses_all_but_last_token():
    o = SlotOracle(2)
    p = np.arange(30)
    _serve(o, p)
    s, r = _serve(o, p)
    assert (s, r) == (0, 29)


def _rotation(n_slots, clients, literal=False, turns=6):
    o = SlotOracle(n_slots, literal_rule=literal)
    order = synth.rotation_sessions(7, clients, turns, 120, 7, 20, 30)
    prev = {}
    rows = []
    for sess, p in order:
        s, r = _serve(o, p)
        rows.append((sess, len(p), r, len(p) - prev.get(sess, 0)))
        prev[sess] = len(p)
    return rows


@pytest.mark.parametrize("clients", [1, 2, 4])
def test_four_slots_prefill_only_the_new_turn(clients):
    """With four slots each conversation keeps its history: from the second
    turn on only the appended tokens are prefilled, at 1, 2 and 4 clients."""
    rows = _rotation(4, clients)
    for i, (sess, n, r, appended) in enumerate(rows):
        if i >= clients:
            assert n - r == appended


def test_one_slot_two_clients_reuses_only_the_header():
    """With one slot and two alternating clients every turn after the first
    reuses only the 7-token shared start."""
    rows = _rotation(1, 2)
    for i, (sess, n, r, appended) in enumerate(rows):
        if i >= 1:
            assert r == 7


def test_one_slot_prefill_grows_with_history():
    rows = _rotation(1, 4)
    later = [n - r for i, (s, n, r, a) in enumerate(rows) if i >= 4]
    per_turn = [later[i] for i in range(0, len(later), 4)]
    assert all(b > a for a, b in zip(per_turn, per_turn[1:]))


def test_literal_rule_thrashes_at_two_clients_and_the_reading_does_not():
    """The one-sentence rule lets the second conversation take the first
    one's lone slot on the strength of the shared header, and the two then
    keep evicting each other (reusing only 7 tokens); with the lone-slot
    clause each conversation keeps its own slot."""
    lit = _rotation(4, 2, literal=True)
    assert all(r == 7 for i, (_, _, r, _) in enumerate(lit) if i >= 1)
    ours = _rotation(4, 2, literal=False)
    assert all(n - r == a for i, (_, n, r, a) in enumerate(ours) if i >= 2)


def test_lru_eviction_cuts_back_to_shared_point():
    o = SlotOracle(2)
    hdr = [9, 9, 9]
    a = np.array(hdr + [1] * 10)
    b = np.array(hdr + [2] * 10)
    c = np.array(hdr + [3] * 10)
    assert _serve(o, a) == (0, 0)
    assert _serve(o, b) == (1, 0)
    s, r = _serve(o, c)          # no eligible slot, no empty slot: LRU (slot 0)
    assert (s, r) == (0, 3)


def test_truncate_then_extend_refills():
    o = SlotOracle(1, n_layers=2)
    p = np.arange(20)
    _serve(o, p)
    o.truncate(0, 12)
    assert o.kv_len[0] == [12, 12]
    assert o.extend(0, 1, 8) == 12
    with pytest.raises(ValueError):
        o.extend(0, 1, 1)
    with pytest.raises(ValueError):
        o.truncate(0, 13)        # layer 0 holds only 12 rows


def test_selected_slot_is_claimed_before_prefill():
    """Prompts placed before any prefill get distinct slots: a slot handed to
    a conversation is no longer empty ('How it works': a new conversation
    takes an empty slot, else the least recently used one)."""
    o = SlotOracle(4)
    got = [o.select(np.array([9, 9, 9, s, s])) for s in range(4)]
    assert got == [(0, 0), (1, 0), (2, 0), (3, 0)]
    assert o.select(np.array([9, 9, 9, 7])) == (0, 0)   # LRU; nothing resident yet
