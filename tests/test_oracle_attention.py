"""Pins of the extend-attention oracle: brute force, invariants fixed by the
pages, closed forms and an independent library routine (CPU only)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle.attention import (attention_bytes, attention_flops, extend_attention,
                              extend_attention_bruteforce)


def _case(seed, hq, hkv, d, prefix, m):
    c = synth.attention_case(seed, hq, hkv, d, prefix, m)
    k = np.concatenate([c["k_prefix"], c["k"]])
    v = np.concatenate([c["v_prefix"], c["v"]])
    return c, k, v


@pytest.mark.parametrize("prefix,m", [(0, 1), (0, 4), (3, 1), (5, 3), (2, 6)])
def test_bruteforce_matches_vectorised(prefix, m):
    c, k, v = _case(1, 4, 2, 8, prefix, m)
    a = extend_attention(c["q"], k, v, prefix)
    b = extend_attention_bruteforce(c["q"], k, v, prefix)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_extend_equals_tail_of_full_prefill():
    """Prefilling only the suffix against the cached prefix gives the last
    rows of a from-scratch prefill (goinfer, 'Turn nine in under half a
    second', 'What goinfer does'; openjev 'Latency', 'Accuracy': reuse only
    changes summation order)."""
    P, m = 37, 11
    c, k, v = _case(2, 6, 2, 16, P, m)
    q_all = np.concatenate([c["q_prefix"], c["q"]])
    full = extend_attention(q_all, k, v, 0)
    ext = extend_attention(c["q"], k, v, P)
    assert np.allclose(full[P:], ext, rtol=0, atol=1e-12)


def test_token_by_token_equals_one_pass():
    """m calls with one row each equal one call with m rows (the decode vs
    prefill agreement whose absence the goinfer page reports in 'What we got
    wrong', the one-token-short bug)."""
    P, m = 20, 9
    c, k, v = _case(3, 4, 4, 8, P, m)
    one = extend_attention(c["q"], k, v, P)
    rows = [extend_attention(c["q"][i:i + 1], k[:P + i + 1], v[:P + i + 1], P + i)[0]
            for i in range(m)]
    assert np.allclose(np.stack(rows), one, rtol=0, atol=1e-12)


def test_split_suffix_anywhere():
    P, m = 13, 10
    c, k, v = _case(4, 4, 1, 8, P, m)
    one = extend_attention(c["q"], k, v, P)
    for cut in (1, 4, 9):
        a = extend_attention(c["q"][:cut], k[:P + cut], v[:P + cut], P)
        b = extend_attention(c["q"][cut:], k, v, P + cut)
        assert np.allclose(np.concatenate([a, b]), one, rtol=0, atol=1e-12)


def test_single_visible_key_returns_its_value():
    c, k, v = _case(5, 4, 2, 8, 0, 3)
    o = extend_attention(c["q"], k, v, 0)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    assert np.array_equal(o[0, 0], vf[0, 0]) and np.array_equal(o[0, 3], vf[0, 1])


def test_equal_keys_give_mean_of_visible_values():
    """With all keys equal every visible key gets the same weight, so each
    row's output is the mean of the values it can see; this also fixes the
    GQA map (q head h reads KV head h // g)."""
    P, m, hq, hkv, d = 6, 4, 6, 3, 8
    c, k, v = _case(6, hq, hkv, d, P, m)
    k = np.broadcast_to(k[:1], k.shape).copy()
    o = extend_attention(c["q"], k, v, P)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    for i in range(m):
        for h in range(hq):
            assert np.allclose(o[i, h], vf[:P + i + 1, h // (hq // hkv)].mean(axis=0),
                               rtol=0, atol=1e-12)


def test_zero_query_gives_mean():
    P, m = 4, 2
    c, k, v = _case(7, 2, 1, 8, P, m)
    q = np.zeros_like(c["q"])
    o = extend_attention(q, k, v, P)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    assert np.allclose(o[1, 0], vf[:P + 2, 0].mean(axis=0), rtol=0, atol=1e-12)


def test_score_scale_is_inverse_sqrt_d():
    """Two keys with q.k = 0 and q.k = 2 at D = 4: scores 0 and 2/sqrt(4) = 1,
    so the weights are 1/(1+e) and e/(1+e)."""
    d = 4
    q = np.zeros((1, 1, d), np.float32); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, d), np.float32); k[1, 0, 0] = 2.0
    v = np.zeros((2, 1, d), np.float32); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    o = extend_attention(synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k),
                         synth.f32_to_bf16_bits(v), 1)
    e = math.e
    assert o[0, 0, 1] == pytest.approx(1 / (1 + e), abs=1e-15)
    assert o[0, 0, 2] == pytest.approx(e / (1 + e), abs=1e-15)


def test_empty_suffix_is_noop():
    c, k, v = _case(8, 2, 1, 8, 5, 1)
    o = extend_attention(c["q"][:0], k[:5], v[:5], 5)
    assert o.shape == (0, 2, 8)


def test_matches_torch_sdpa_float64():
    """Independent library routine: torch's scaled_dot_product_attention on
    the CPU in float64 with an explicit offset-causal mask and repeated KV."""
    P, m, hq, hkv, d = 50, 17, 8, 2, 32
    c, k, v = _case(9, hq, hkv, d, P, m)
    o = extend_attention(c["q"], k, v, P)
    q = torch.from_numpy(synth.bf16_bits_to_f32(c["q"]).astype(np.float64)).permute(1, 0, 2)
    kk = torch.from_numpy(synth.bf16_bits_to_f32(k).astype(np.float64)).permute(1, 0, 2)
    vv = torch.from_numpy(synth.bf16_bits_to_f32(v).astype(np.float64)).permute(1, 0, 2)
    g = hq // hkv
    kk = kk.repeat_interleave(g, dim=0)
    vv = vv.repeat_interleave(g, dim=0)
    mask = torch.arange(P + m)[None, :] <= (P + torch.arange(m))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# planted mistakes in the oracle's definition: each must fail a pin above
def _mutant_no_offset(q, k, v, prefix):
    # row i sees keys 0..i instead of 0..prefix+i
    return extend_attention(q, k[:q.shape[0]] if prefix else k, v[:q.shape[0]] if prefix else v, 0)


def test_pins_catch_missing_causal_offset():
    P, m = 37, 11
    c, k, v = _case(2, 6, 2, 16, P, m)
    q_all = np.concatenate([c["q_prefix"], c["q"]])
    full = extend_attention(q_all, k, v, 0)
    bad = _mutant_no_offset(c["q"], k, v, P)
    assert not np.allclose(full[P:], bad, atol=1e-3)


def test_work_counts():
    # turn 9 of the 7B-like replay: 1668 cached + 254 new rows, 28 heads, D 128
    assert attention_flops(1668, 254, 28, 128) == 4 * 128 * 28 * (254 * 1668 + 254 * 255 // 2)
    assert attention_flops(1668, 254, 28, 128) == 6_538_033_152
    assert attention_bytes(0, 1, 1, 1, 2) == 2 * 1 * 2 * 2 + 2 * 2 * 2 + 4 * 2 * 2
