"""Pins of the int4 / GEMV oracle against closed forms, exhaustive checks,
brute force and planted mistakes (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import w4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# dequantisation
# --------------------------------------------------------------------------

def test_dequant_hand_worked_fixture():
    """A hand-written block: codes and expected values written out literally."""
    with open(os.path.join(GOLDEN, "w4_block_hand.json")) as f:
        fx = json.load(f)
    w = np.array(fx["bytes"], dtype=np.uint8).reshape(fx["n"], fx["k"] // 2)
    s = np.array(fx["scales_f16"], dtype=np.float16).view(np.uint16).reshape(fx["n"], fx["k"] // 32)
    got = w4.dequant(w, s, fx["k"])
    want = np.array(fx["expected"], dtype=np.float64).reshape(fx["n"], fx["k"])
    assert np.array_equal(got, want)


def test_dequant_rejects_ragged_k():
    with pytest.raises(ValueError):
        w4.dequant(np.zeros((1, 24), np.uint8), np.zeros((1, 1), np.uint16), 48)


def test_dequant_product_exact_in_fp32():
    """(code-8)*scale is exact in fp32 for every code and every finite fp16
    scale, so a GPU dequant to fp32 can be compared bit for bit."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    fin = np.isfinite(h)
    s64 = h[fin].astype(np.float64)
    s32 = h[fin].astype(np.float32)
    for code in range(16):
        p64 = (code - 8) * s64
        p32 = (np.float32(code - 8) * s32).astype(np.float64)
        assert np.array_equal(p64, p32)
    assert fin.sum() == 63488


def test_dequant_nibble_order_and_groups():
    """Element k of row n reads nibble (k&1) of byte k//2 and scale k//32:
    distinct codes and distinct per-group scales make any mix-up visible."""
    n, k = 3, 96
    codes = (np.arange(n * k).reshape(n, k) * 7 + 3) % 16
    w = synth.pack_nibbles(codes)
    sc = (np.arange(n * (k // 32)).reshape(n, k // 32) + 1).astype(np.float16)
    got = w4.dequant(w, sc.view(np.uint16), k)
    for r in range(n):
        for c in range(k):
            assert got[r, c] == (codes[r, c] - 8) * float(sc[r, c // 32])


# --------------------------------------------------------------------------
# GEMV
# --------------------------------------------------------------------------

def _gemv_bruteforce(x_bits, w, s, k):
    x = _bf16_f64(x_bits)
    m, n = x.shape[0], w.shape[0]
    y = np.zeros((m, n))
    for r in range(m):
        for j in range(n):
            terms = []
            for c in range(k):
                byte = int(w[j, c // 2])
                code = (byte >> 4) if c % 2 else (byte & 15)
                sc = float(np.uint16(s[j, c // 32]).view(np.float16))
                terms.append(x[r, c] * (code - 8) * sc)
            y[r, j] = math.fsum(terms)
    return y


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (3, 4, 64), (2, 3, 32)])
def test_gemv_bruteforce(m, n, k):
    g = synth.rng(11, m, n, k)
    w, s = synth.w4_weights(g, n, k)
    x = synth.normal_bf16(g, (m, k))
    got = w4.gemv(x, w, s, k)
    want = _gemv_bruteforce(x, w, s, k)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_gemv_zero_input_gives_zero():
    g = synth.rng(12)
    w, s = synth.w4_weights(g, 16, 64)
    x = np.zeros((4, 64), np.uint16)
    assert np.array_equal(w4.gemv(x, w, s, 64), np.zeros((4, 16)))


def test_gemv_code9_scale1_is_row_sum():
    """All codes 9 and scales 1 make every weight 1: y = sum of the row of x."""
    k, n = 64, 5
    w = synth.pack_nibbles(np.full((n, k), 9))
    s = np.ones((n, k // 32), np.float16).view(np.uint16)
    g = synth.rng(13)
    x = synth.normal_bf16(g, (3, k))
    y = w4.gemv(x, w, s, k)
    rs = np.array([math.fsum(r) for r in _bf16_f64(x)])
    assert np.allclose(y, rs[:, None], rtol=0, atol=1e-12)


def test_gemv_one_hot_reads_one_weight():
    g = synth.rng(14)
    n, k = 8, 96
    w, s = synth.w4_weights(g, n, k)
    dq = w4.dequant(w, s, k)
    for c in (0, 1, 31, 32, 33, 95):
        x = np.zeros((1, k), np.float32)
        x[0, c] = 1.0
        y = w4.gemv(synth.f32_to_bf16_bits(x), w, s, k)
        assert np.array_equal(y[0], dq[:, c])


def test_gemv_rows_independent():
    g = synth.rng(15)
    w, s = synth.w4_weights(g, 40, 128)
    x = synth.normal_bf16(g, (8, 128))
    full = w4.gemv(x, w, s, 128)
    for r in range(8):
        assert np.array_equal(full[r], w4.gemv(x[r:r + 1], w, s, 128)[0])


def test_gemv_chunking_matches_single_product():
    """Column chunking (to bound memory) equals one product of the whole matrix."""
    g = synth.rng(16)
    n, k = 3000, 2048
    w, s = synth.w4_weights(g, n, k)
    x = synth.normal_bf16(g, (2, k))
    y = w4.gemv(x, w, s, k)
    ref = _bf16_f64(x) @ w4.dequant(w, s, k).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-12)


# planted mistakes: each variant of the oracle must fail at least one pin
def _mutants():
    def swapped_nibbles(w, s, k):
        q = w4.nibbles(w, k)
        q = q.reshape(q.shape[0], -1, 2)[:, :, ::-1].reshape(q.shape[0], k)
        return (q - 8) * np.repeat(w4._fp16_to_f64(s), 32, axis=1)

    def zero_point_7(w, s, k):
        return (w4.nibbles(w, k) - 7) * np.repeat(w4._fp16_to_f64(s), 32, axis=1)

    def group_16(w, s, k):
        sc = w4._fp16_to_f64(s)
        idx = np.minimum(np.arange(k) // 16, sc.shape[1] - 1)
        return (w4.nibbles(w, k) - 8) * sc[:, idx]

    def sign_flip(w, s, k):
        return (8 - w4.nibbles(w, k)) * np.repeat(w4._fp16_to_f64(s), 32, axis=1)

    return [swapped_nibbles, zero_point_7, group_16, sign_flip]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_dequant_mistakes(mutant):
    with open(os.path.join(GOLDEN, "w4_block_hand.json")) as f:
        fx = json.load(f)
    w = np.array(fx["bytes"], dtype=np.uint8).reshape(fx["n"], fx["k"] // 2)
    s = np.array(fx["scales_f16"], dtype=np.float16).view(np.uint16).reshape(fx["n"], fx["k"] // 32)
    want = np.array(fx["expected"], dtype=np.float64).reshape(fx["n"], fx["k"])
    assert not np.array_equal(mutant(w, s, fx["k"]), want)


# --------------------------------------------------------------------------
# routed GEMV and distinct-expert accounting
# --------------------------------------------------------------------------

def test_routed_reduces_to_dense_per_pair():
    g = synth.rng(21)
    e_all, n, k, m, topk = 6, 16, 64, 3, 2
    ws = [synth.w4_weights(g, n, k) for _ in range(e_all)]
    w_all = np.stack([a for a, _ in ws])
    s_all = np.stack([b for _, b in ws])
    ids, _ = synth.routing_topk(g, m, e_all, topk)
    x = synth.normal_bf16(g, (m, k))
    y = w4.gemv_routed(x, False, ids, w_all, s_all, k)
    xs = synth.normal_bf16(g, (m, topk, k))
    ys = w4.gemv_routed(xs, True, ids, w_all, s_all, k)
    for r in range(m):
        for j in range(topk):
            e = ids[r, j]
            assert np.array_equal(y[r, j], w4.gemv(x[r:r + 1], w_all[e], s_all[e], k)[0])
            assert np.array_equal(ys[r, j], w4.gemv(xs[r, j][None], w_all[e], s_all[e], k)[0])


def test_routed_rejects_bad_expert():
    g = synth.rng(22)
    w, s = synth.w4_weights(g, 4, 32)
    with pytest.raises(ValueError):
        w4.gemv_routed(np.zeros((1, 32), np.uint16), False, np.array([[3]]),
                       w[None], s[None], 32)


def test_topk_routing_is_top_logits():
    g = synth.rng(23)
    ids, logits = synth.routing_topk(g, 8, 256, 8)
    for r in range(8):
        assert len(set(ids[r])) == 8
        thr = np.sort(logits[r])[-8]
        assert all(logits[r, e] >= thr for e in ids[r])


def test_distinct_expert_count_bruteforce():
    ids = np.array([[1, 2, 3], [3, 4, 1], [9, 2, 4]])
    assert w4.distinct_experts(ids) == 5  # {1, 2, 3, 4, 9}


def test_expected_distinct_matches_simulation():
    """E[union] = E (1 - (1 - k/E)^m) against seeded draws."""
    g = synth.rng(24)
    for m in (1, 2, 4, 8):
        sims = []
        for _ in range(400):
            ids, _ = synth.routing_topk(g, m, 256, 8)
            sims.append(w4.distinct_experts(ids))
        mean = float(np.mean(sims))
        se = float(np.std(sims)) / math.sqrt(len(sims)) + 1e-9
        assert abs(mean - w4.expected_distinct(m, 256, 8)) < 5 * se + 1e-9
    assert w4.expected_distinct(1, 256, 8) == pytest.approx(8.0)


def test_byte_counts():
    # one 9B-like fused gate||up matrix: 24576 x 4096 at 4.5 bits per weight
    assert w4.expert_bytes(24576, 4096) == 24576 * 4096 * 9 // 16
    assert w4.gemv_bytes(1, 32, 64) == 32 * 32 + 32 * 2 * 2 + 2 * 64 + 4 * 32
