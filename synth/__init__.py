"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and bench.py.

This module only draws random numbers and lays them out in the storage formats
the library consumes (bf16 / fp16 bit patterns, packed nibbles, token lists).
It holds none of the method's arithmetic: no attention, no dequantisation, no
matrix products, no slot matching.

Storage formats produced here:
  * bf16 tensors as uint16 bit patterns (round-to-nearest-even from fp32 draws);
  * fp16 scales as uint16 bit patterns (numpy's float16 cast, nearest-even);
  * int4 weights as uint8 [N][K/2]: byte k//2 of row n holds element k in its
    low nibble when k is even and in its high nibble when k is odd;
  * token ids as int32.

Workload shapes follow the five single-layer workloads this library is
measured on (see ``WORKLOADS``).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# workloads (shapes only)
# --------------------------------------------------------------------------

WORKLOADS = {
    # tiny single layer: fast enough for the oracle in well under a second
    "tiny": dict(hidden=256, hq=4, hkv=2, d=64, prefix=64, m=8,
                 gemv_n=1024, gemv_k=256, seed=0),
    # agent-turn replay, 7B-like attention layer; prompt lengths of the
    # ten-turn replay (turn 10's length is an extrapolation of the step)
    "replay7b": dict(hidden=3584, hq=28, hkv=4, d=128, ffn=18944,
                     prompt_lengths=(727, 861, 996, 1130, 1265, 1399, 1534,
                                     1668, 1922, 2056), seed=2),
    # speculative verify sweep, 9B-like dense layer
    "verify9b": dict(hidden=4096, hq=32, hkv=8, d=128, ffn=12288,
                     context=2048, m_values=tuple(range(1, 9)), seed=3),
    # MoE verify, 35B-A3B-like expert layer
    "moe35b": dict(hidden=2048, n_experts=256, expert_ffn=512, topk=8,
                   m_values=tuple(range(1, 9)), seed=4),
    # four resident slots in rotation, 4B-like attention layer
    "slots4b": dict(hidden=2560, hq=32, hkv=8, d=128, n_slots=4,
                    state_tokens=800, shared_start=7, turns=6,
                    question_min=24, question_max=36, seed=5),
}


def layer_gemv_shapes(hidden: int, ffn: int, hq: int, hkv: int, d: int):
    """(N, K) of the four int4 projections of one dense decoder layer:
    fused QKV, attention output, fused gate||up, down."""
    qkv = (hq + 2 * hkv) * d
    return [(qkv, hidden), (hq * d, hidden), (2 * ffn, hidden), (hidden, ffn)]


# --------------------------------------------------------------------------
# bit-pattern helpers (storage only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def fp16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen float16 bit patterns to float32 (exact)."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[N][K] integers 0..15 -> uint8 [N][K/2], even k in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    assert nib.ndim == 2 and nib.shape[1] % 2 == 0
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------

def rng(seed: int, *stream: int) -> np.random.Generator:
    """Independent PCG64 stream per (seed, stream...)."""
    return np.random.default_rng([seed, *stream])


def normal_bf16(g: np.random.Generator, shape) -> np.ndarray:
    """bf16 bits of N(0,1) draws."""
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32))


def w4_weights(g: np.random.Generator, n: int, k: int,
               scale_lo: float = 0.01, scale_hi: float = 0.05):
    """Random int4 group-32 weight: (packed uint8 [n][k/2], fp16 bits [n][k/32]).

    Nibbles uniform on 0..15 (zero point 8), scales fp16 of U(lo, hi)."""
    assert k % 32 == 0
    nib = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    scales = g.uniform(scale_lo, scale_hi, size=(n, k // 32)).astype(np.float16)
    return pack_nibbles(nib), scales.view(np.uint16)


def routing_topk(g: np.random.Generator, m: int, n_experts: int, topk: int):
    """Top-k expert ids per row from U(0,1) float32 logits.

    Ids are sorted by descending logit; equal logits keep the lower id first.
    Returns (ids int32 [m][topk], logits float32 [m][n_experts])."""
    logits = g.random((m, n_experts), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    return order.astype(np.int32), logits


def tokens(g: np.random.Generator, n: int, vocab: int = 65536) -> np.ndarray:
    return g.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------
# conversation scenarios for the slot matcher
# --------------------------------------------------------------------------

def rotation_sessions(seed: int, n_sessions: int, turns: int, state_tokens: int,
                      shared_start: int, question_min: int, question_max: int,
                      vocab: int = 65536):
    """Prompts of ``n_sessions`` conversations taking turns round-robin.

    Every conversation starts with the same ``shared_start`` tokens (the
    chat-template header), then ``state_tokens - shared_start`` tokens of its
    own; each turn appends a question of U{question_min..question_max} tokens.
    Returns the request order as a list of (session, prompt int32 array)."""
    g = rng(seed, 101)
    header = tokens(g, shared_start, vocab)
    prompts = []
    for _ in range(n_sessions):
        body = tokens(g, state_tokens - shared_start, vocab)
        prompts.append(np.concatenate([header, body]))
    order = []
    for _t in range(turns):
        for s in range(n_sessions):
            q = tokens(g, int(g.integers(question_min, question_max + 1)), vocab)
            prompts[s] = np.concatenate([prompts[s], q])
            order.append((s, prompts[s].copy()))
    return order


def replay_prompt(seed: int, lengths, vocab: int = 65536):
    """Token prompts of a growing agent replay: each prompt extends the last."""
    g = rng(seed, 102)
    full = tokens(g, int(max(lengths)), vocab)
    return [full[:L].copy() for L in lengths]


# --------------------------------------------------------------------------
# attention rows
# --------------------------------------------------------------------------

def attention_rows(g: np.random.Generator, m: int, hq: int, hkv: int, d: int):
    """New rows of one extend call: bf16 bits of N(0,1) q [m][hq][d],
    k [m][hkv][d], v [m][hkv][d] (drawn in the order k, v, q)."""
    k = normal_bf16(g, (m, hkv, d))
    v = normal_bf16(g, (m, hkv, d))
    q = normal_bf16(g, (m, hq, d))
    return q, k, v


def attention_case(seed: int, hq: int, hkv: int, d: int, prefix: int, m: int):
    """A cached prefix of ``prefix`` rows followed by ``m`` new rows.

    Returns dict with q_prefix/k_prefix/v_prefix (the rows that filled the
    cache) and q/k/v (the suffix rows), all bf16 bit patterns."""
    gp = rng(seed, 1)
    qp, kp, vp = attention_rows(gp, prefix, hq, hkv, d)
    gs = rng(seed, 2)
    q, k, v = attention_rows(gs, m, hq, hkv, d)
    return dict(q_prefix=qp, k_prefix=kp, v_prefix=vp, q=q, k=k, v=v)


# --------------------------------------------------------------------------
# verify logits
# --------------------------------------------------------------------------

VERIFY_VOCAB = 151936  # a Qwen-family vocabulary size; the pages' models use one


def verify_case(seed: int, m: int, vocab: int, n_match: int, tie: bool = False):
    """Logits and drafts of one verify step of m = k + 1 rows.

    logits: fp32 [m][vocab] drawn N(0,1), then one entry per row set to 8.0 at
    a random id (the planted top entry); with ``tie`` a second random id of
    the row gets the same 8.0. drafts: int32 [m-1], equal to row i's first
    planted id for i < n_match and a different random id after that.
    Returns (logits, drafts, planted ids [m][1 or 2])."""
    g = rng(seed, 7)
    logits = g.standard_normal((m, vocab), dtype=np.float32)
    npl = 2 if tie else 1
    planted = np.stack([g.choice(vocab, size=npl, replace=False) for _ in range(m)])
    for i in range(m):
        logits[i, planted[i]] = np.float32(8.0)
    drafts = np.empty(m - 1, dtype=np.int32)
    for i in range(m - 1):
        if i < n_match:
            drafts[i] = planted[i, 0]
        else:
            d = int(g.integers(0, vocab))
            while d in planted[i]:
                d = int(g.integers(0, vocab))
            drafts[i] = d
    return logits, drafts, planted
