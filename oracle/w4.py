"""Oracle: int4 group-32 weights, the m-row GEMV and the routed (MoE) GEMV.

Test infrastructure only (see ``oracle/__init__.py``).

Storage format (a reading: the pages name the group-32 block formats but not
a byte order): weights are uint8 [N][K/2], byte k//2 of row n holding element
k in its low nibble for even k and its high nibble for odd k; scales are fp16
bit patterns [N][K/32], one per 32 consecutive k of a row; the zero point is 8.
"""
from __future__ import annotations

import numpy as np


def _fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def nibbles(w: np.ndarray, k: int) -> np.ndarray:
    """Integer codes 0..15 of a [N][K/2] packed weight, as int64 [N][K]."""
    w = np.asarray(w, dtype=np.uint8)
    n = w.shape[0]
    assert w.shape == (n, k // 2)
    idx = np.arange(k)
    byte = w[:, idx >> 1].astype(np.int64)
    return (byte >> (4 * (idx & 1))) & 0xF


def dequant(w: np.ndarray, scales: np.ndarray, k: int) -> np.ndarray:
    """fp64 [N][K] value of an int4 group-32 weight.

    Each element is (code - 8) times the fp16 scale of its 32-element group.
    The pages ("Models and quantizations", section "Quantizations") describe
    32-element blocks with a per-block scale used in place, never expanded on
    load; this is the plain group-32 / zero-point-8 form of such a block.
    Raises ValueError unless K is a multiple of 32."""
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    q = nibbles(w, k)
    s = _fp16_to_f64(scales)
    assert s.shape == (q.shape[0], k // 32)
    return (q - 8).astype(np.float64) * np.repeat(s, 32, axis=1)


def gemv(x_bits: np.ndarray, w: np.ndarray, scales: np.ndarray, k: int) -> np.ndarray:
    """y[r, n] = sum_k x[r, k] * w[n, k] in fp64, for bf16 x [m][K], any m.

    The m rows go through the same weight matrix (thinkspread, "The economics
    of speculative decoding", opening section: verify rows share one read of
    the weights; goinfer, "Turn nine in under half a second", section "The
    problem": a prefill runs each new prompt token through every weight);
    the result is the ordinary product of each row with the dequantised
    matrix, the reference of both the m-row GEMV and the many-row GEMM.
    Computed in column chunks to bound memory."""
    x = _bf16_to_f64(x_bits)
    assert x.ndim == 2 and x.shape[1] == k
    n = w.shape[0]
    y = np.empty((x.shape[0], n), dtype=np.float64)
    chunk = max(1, (1 << 22) // k)
    for n0 in range(0, n, chunk):
        n1 = min(n, n0 + chunk)
        y[:, n0:n1] = x @ dequant(w[n0:n1], scales[n0:n1], k).T
    return y


def gemv_routed(x_bits: np.ndarray, x_per_slot: bool, expert_ids: np.ndarray,
                w_all: np.ndarray, s_all: np.ndarray, k: int) -> np.ndarray:
    """Routed GEMV: y[r, j, :] = W_{e(r,j)} x(r, j).

    Each row picks its own experts, so rows do not share expert weights
    (thinkspread, "The economics of speculative decoding", section
    "Architecture decides whether it pays"). x is [m][K] (every expert slot
    of a row sees the row's input) or, with ``x_per_slot``, [m][topk][K].
    w_all [E][N][K/2], s_all [E][N][K/32]; returns fp64 [m][topk][N]."""
    ids = np.asarray(expert_ids)
    m, topk = ids.shape
    e_all, n = w_all.shape[0], w_all.shape[1]
    y = np.empty((m, topk, n), dtype=np.float64)
    cache = {}
    for r in range(m):
        for j in range(topk):
            e = int(ids[r, j])
            if not 0 <= e < e_all:
                raise ValueError("expert id out of range")
            if e not in cache:
                cache[e] = dequant(w_all[e], s_all[e], k)
            xr = x_bits[r, j] if x_per_slot else x_bits[r]
            y[r, j] = _bf16_to_f64(xr[None, :]) @ cache[e].T
    return y


def expert_bytes(n: int, k: int) -> int:
    """Bytes of one int4 group-32 expert matrix: K/2 nibble bytes plus K/32
    fp16 scales per row."""
    return n * (k // 2) + n * (k // 32) * 2


def distinct_experts(expert_ids: np.ndarray) -> int:
    """Number of distinct experts the m rows route to: each is read once
    when its weights are shared among the rows that chose it."""
    return len(set(int(e) for e in np.asarray(expert_ids).ravel()))


def expected_distinct(m: int, n_experts: int, topk: int) -> float:
    """E[#distinct experts] when each of m rows draws ``topk`` distinct
    experts uniformly: n_experts * (1 - (1 - topk/n_experts)^m)."""
    return n_experts * (1.0 - (1.0 - topk / n_experts) ** m)


def gemv_bytes(m: int, n: int, k: int) -> int:
    """Algorithmic bytes of one m-row GEMV call: the int4 weights and fp16
    scales once, bf16 x, fp32 y."""
    return n * (k // 2) + n * (k // 32) * 2 + 2 * m * k + 4 * m * n
