"""GPU slot selection (LCP kernel + host rule) is bit-exact with the oracle:
the same (slot, reused) for every request of seeded conversation scenarios
and of random small-alphabet prompts, under both matching rules and with
reuse off; the memory check grants fewer slots when the arena is short."""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle.slots import SlotOracle
from tests.gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu
HQ, HKV, D = 1, 1, 64


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _fill(st, slot, n):
    """Prefill the rest of the selected prompt (rows are arbitrary here)."""
    m = n - st.kv_len(slot)
    if m:
        q = torch.zeros((m, HQ, D), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((m, HKV, D), dtype=torch.bfloat16, device="cuda")
        st.extend_attn(slot, 0, q, k, k)


def _compare(requests, n_slots, reuse=True, literal=False, cap=2048):
    st = sve.KVSlots(n_slots, 1, HQ, HKV, D, cap, cap, reuse=reuse,
                     match_rule=1 if literal else 0)
    o = SlotOracle(n_slots, reuse=reuse, literal_rule=literal)
    for idx, p in enumerate(requests):
        got = st.kv_slot_select(p)
        want = o.select(p)
        assert got == want, (idx, got, want)
        _fill(st, got[0], len(p))
        for layer in range(o.n_layers):
            o.extend(want[0], layer, len(p) - o.kv_len[want[0]][layer])
    return st


@pytest.mark.parametrize("clients", [1, 2, 4])
@pytest.mark.parametrize("n_slots", [1, 4])
def test_rotation_scenarios(n_slots, clients):
    announce(f"rotation slots={n_slots} clients={clients}")
    order = synth.rotation_sessions(5, clients, 6, 200, 7, 24, 36)
    _compare([p for _, p in order], n_slots)


def test_literal_rule_and_reuse_off():
    order = [p for _, p in synth.rotation_sessions(6, 2, 5, 120, 7, 24, 36)]
    announce("literal / reuse off")
    _compare(order, 4, literal=True)
    _compare(order, 4, reuse=False)


def test_random_small_alphabet_prompts():
    """Prompts built from a few shared stems over a 3-token alphabet, so
    common prefixes of every length and ties between slots occur often."""
    g = synth.rng(7)
    stems = [g.integers(0, 3, size=int(g.integers(1, 12))).astype(np.int32) for _ in range(6)]
    reqs = []
    for _ in range(300):
        a = stems[int(g.integers(0, 6))]
        tail = g.integers(0, 3, size=int(g.integers(0, 8))).astype(np.int32)
        p = np.concatenate([a, tail])
        if len(p) == 0:
            p = np.array([1], np.int32)
        reqs.append(p)
    announce("random prompts")
    for n_slots in (2, 3, 4):
        _compare(reqs, n_slots)
        _compare(reqs, n_slots, literal=True)


def test_long_prompts_cross_kernel_chunks():
    """Common prefixes longer than one 1024-token scan chunk."""
    base = synth.tokens(synth.rng(8), 3000)
    reqs = [base[:2500], base[:2600], np.concatenate([base[:1500], [7, 7, 7]]), base[:2700]]
    announce("long prompts")
    _compare(reqs, 2, cap=4096)


def test_granted_slots_follow_arena_size():
    st4 = sve.KVSlots(4, 2, 8, 2, 64, 256, 64)
    need = st4.arena.numel()
    per_slot = 2 * 2 * (2 * 256 * 64 * 2)
    short = need - per_slot  # room for three slots
    announce("granted slots")
    st3 = sve.KVSlots(4, 2, 8, 2, 64, 256, 64, arena_bytes=short)
    assert (st4.granted, st3.granted) == (4, 3)


def test_select_rejects_bad_prompts():
    st = sve.KVSlots(2, 1, HQ, HKV, D, 128, 64)
    with pytest.raises(sve.SveError):
        st.kv_slot_select(np.zeros(0, np.int32))
    with pytest.raises(sve.SveError) as e:
        st.kv_slot_select(np.zeros(129, np.int32))
    assert e.value.code == -3


def test_batch_placement_before_prefill():
    """Four prompts selected before one batched extend land in four slots,
    as in the oracle; the rotation then reuses each slot's history."""
    order = synth.rotation_sessions(9, 4, 3, 100, 7, 24, 36)
    st = sve.KVSlots(4, 1, HQ, HKV, D, 1024, 1024)
    o = SlotOracle(4)
    announce("batch placement")
    for rnd in range(3):
        reqs = [p for _, p in order[4 * rnd:4 * rnd + 4]]
        got = [st.kv_slot_select(p) for p in reqs]
        want = [o.select(p) for p in reqs]
        assert got == want
        assert len({s for s, _ in got}) == 4
        for (s, r), p in zip(got, reqs):
            _fill(st, s, len(p))
            o.extend(s, 0, len(p) - o.kv_len[s][0])
        if rnd:
            assert all(r > 0 for _, r in got)
