"""Oracle: extend-prefill attention.

Test infrastructure only (see ``oracle/__init__.py``).

A cached prefix of P positions is kept (goinfer, "Turn nine in under half a
second", sections "What goinfer does" and "How it works": the KV cache stores
a key and a value vector per token and layer, and only the tokens after the
reused start are prefilled). The m new rows are the positions P..P+m-1; row i
attends causally to positions 0..P+i.

Readings where the pages are silent (each is listed in the design doc):
  * scores are scaled by 1/sqrt(D);
  * no rotary embedding inside the operation: q and k arrive position-encoded;
  * grouped-query attention: q head h reads KV head h // (Hq / Hkv);
  * row i sees keys 0..P+i inclusive; no soft-cap, window or bias;
  * m == 0 is a no-op, P == 0 is a full prefill.

Layouts: q [m][Hq][D], k and v [P+m][Hkv][D] (the whole visible sequence),
all bf16 bit patterns; outputs fp64 [m][Hq][D].
"""
from __future__ import annotations

import math

import numpy as np


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def extend_attention(q_bits, k_bits, v_bits, prefix: int) -> np.ndarray:
    """softmax(q k^T / sqrt(D)) v over the causally visible keys, in fp64.

    For query row i (absolute position prefix + i) and head h:
        s_j = q[i,h] . k[j, h // g] / sqrt(D),  j = 0 .. prefix + i
        o[i,h] = sum_j exp(s_j - max s) v[j, h // g] / sum_j exp(s_j - max s)
    """
    q = _bf16_to_f64(q_bits)
    k = _bf16_to_f64(k_bits)
    v = _bf16_to_f64(v_bits)
    m, hq, d = q.shape
    t, hkv, d2 = k.shape
    assert d2 == d and v.shape == k.shape and t == prefix + m
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    out = np.zeros((m, hq, d), dtype=np.float64)
    if m == 0:
        return out
    pos = prefix + np.arange(m)                     # absolute query positions
    visible = np.arange(t)[None, :] <= pos[:, None]  # [m][t]
    for h in range(hq):
        kh = k[:, h // g, :]
        vh = v[:, h // g, :]
        s = (q[:, h, :] @ kh.T) / math.sqrt(d)       # [m][t]
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, h, :] = (p @ vh) / p.sum(axis=1, keepdims=True)
    return out


def extend_attention_bruteforce(q_bits, k_bits, v_bits, prefix: int) -> np.ndarray:
    """The same definition with explicit loops and exactly rounded sums
    (math.fsum); for tiny shapes only."""
    q = _bf16_to_f64(q_bits)
    k = _bf16_to_f64(k_bits)
    v = _bf16_to_f64(v_bits)
    m, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((m, hq, d), dtype=np.float64)
    for i in range(m):
        last = prefix + i
        for h in range(hq):
            kv = h // g
            s = [math.fsum(q[i, h, c] * k[j, kv, c] for c in range(d)) / math.sqrt(d)
                 for j in range(last + 1)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            den = math.fsum(e)
            for c in range(d):
                out[i, h, c] = math.fsum(e[j] * v[j, kv, c] for j in range(last + 1)) / den
    return out


def extend_attention_questions(q_bits, k_prefix_bits, v_prefix_bits, k_new_bits, v_new_bits,
                               ms) -> np.ndarray:
    """Several questions about one cached state (openjev-multimodal,
    "Latency", section "What changed": with prefix priming the shared prefix
    is evaluated once and each question resumes from that checkpoint,
    reading only its own text).

    The question rows are packed question after question (ms[j] rows each):
    q [sum m][Hq][D], k_new / v_new [sum m][Hkv][D]; the prefix is
    k_prefix / v_prefix [P][Hkv][D]. Question j is an ordinary extend of the
    prefix by its own rows, so its row i sees prefix positions 0..P-1 and its
    own rows 0..i, never another question's. Returns fp64 [sum m][Hq][D]."""
    kp = np.asarray(k_prefix_bits)
    vp = np.asarray(v_prefix_bits)
    prefix = kp.shape[0]
    out, r = [], 0
    for m in ms:
        rows = slice(r, r + int(m))
        kk = np.concatenate([kp, np.asarray(k_new_bits)[rows]])
        vv = np.concatenate([vp, np.asarray(v_new_bits)[rows]])
        out.append(extend_attention(np.asarray(q_bits)[rows], kk, vv, prefix))
        r += int(m)
    return np.concatenate(out) if out else np.zeros((0,) + np.asarray(q_bits).shape[1:])


def attention_flops(prefix: int, m: int, hq: int, d: int) -> int:
    """Algorithmic flops of one extend call: 2*D multiply-adds for q.k and
    2*D for p.v per visible (row, key) pair and query head."""
    pairs = m * prefix + m * (m + 1) // 2
    return 4 * d * hq * pairs


def attention_bytes(prefix: int, m: int, hq: int, hkv: int, d: int) -> int:
    """Algorithmic bytes of one extend call: the K and V of all P+m visible
    positions read once (bf16), q read, out written (bf16), and the m new K
    and V rows read and stored."""
    kv = 2 * (prefix + m) * hkv * d * 2
    return kv + 2 * m * hq * d * 2 + 2 * 2 * m * hkv * d * 2
