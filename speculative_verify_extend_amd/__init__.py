"""Extend-prefill attention over resident KV slots and the m-row int4 GEMV on
AMD Instinct MI355X (gfx950).

Thin torch-facing binding of libsve (include/sve.h): it checks tensor
devices, dtypes and shapes, passes raw pointers and the current HIP stream,
and nothing else. Every computation runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib
from ._lib import SveError, check

__all__ = ["KVSlots", "ngram_draft", "w4_packed_bytes", "w4_pack", "w4_dequant", "w4_gemv_m", "w4_gemm",
           "w4_gemm_workspace_bytes",
           "w4_gemv_m_routed", "verify_workspace_bytes", "verify_accept", "verify_accept_noalloc",
           "SpecGate",
           "spec_break_even", "probe_read", "probe_copy", "probe_compute", "SveError", "load_library"]


def load_library():
    """Load libsve.so (raises if it was not built)."""
    return _lib.load()


def _stream() -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor) -> C.c_void_p:
    return C.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, dtype, shape, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class KVSlots:
    """A resident KV-slot store (up to four conversations) on one GPU."""

    def __init__(self, n_slots: int, n_layers: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, capacity: int, max_rows: int, reuse: bool = True,
                 match_rule: int = 0, device="cuda", arena_bytes: int | None = None):
        lib = _lib.load()
        self.cfg = _lib.SveConfig(n_slots, n_layers, n_q_heads, n_kv_heads, head_dim,
                                  capacity, max_rows, int(bool(reuse)), match_rule)
        need = lib.sve_arena_bytes(C.byref(self.cfg), n_slots)
        if need == 0:
            raise ValueError("invalid KV-slot configuration")
        nbytes = need if arena_bytes is None else int(arena_bytes)
        self.requested = n_slots
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device)
        ctx = C.c_void_p()
        granted = C.c_int32()
        check(lib.sve_create(C.byref(self.cfg), _ptr(self.arena), nbytes, _stream(),
                             C.byref(ctx), C.byref(granted)))
        self._lib = lib
        self.ctx = ctx
        self.granted = granted.value
        cap = C.c_int32()
        check(lib.sve_info(ctx, C.byref(granted), C.byref(cap)), ctx)
        self.capacity = cap.value
        self.hq, self.hkv, self.d = n_q_heads, n_kv_heads, head_dim

    def close(self) -> None:
        if getattr(self, "ctx", None):
            self._lib.sve_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _bind(self) -> None:
        check(self._lib.sve_set_stream(self.ctx, _stream()), self.ctx)

    def kv_slot_select(self, tokens) -> tuple[int, int]:
        """(slot, reused) for a prompt of token ids (host ints). Synchronises."""
        self._bind()
        arr = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        slot, reused = C.c_int32(), C.c_int32()
        check(self._lib.sve_kv_slot_select(self.ctx, arr.ctypes.data_as(C.c_void_p), arr.size,
                                           C.byref(slot), C.byref(reused)), self.ctx)
        return slot.value, reused.value

    def kv_truncate(self, slot: int, length: int) -> None:
        check(self._lib.sve_kv_truncate(self.ctx, slot, length), self.ctx)

    def kv_len(self, slot: int, layer: int = 0) -> int:
        n = C.c_int32()
        check(self._lib.sve_kv_len(self.ctx, slot, layer, C.byref(n)), self.ctx)
        return n.value

    def extend_attn(self, slot: int, layer: int, q: torch.Tensor, new_k: torch.Tensor,
                    new_v: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """Append m rows to (slot, layer) and attend; q [m][Hq][D] bf16,
        new_k/new_v [m][Hkv][D] bf16; returns out [m][Hq][D] bf16."""
        m = q.shape[0]
        _need(q, torch.bfloat16, (m, self.hq, self.d), "q")
        _need(new_k, torch.bfloat16, (m, self.hkv, self.d), "new_k")
        _need(new_v, torch.bfloat16, (m, self.hkv, self.d), "new_v")
        if out is None:
            out = torch.empty_like(q)
        _need(out, torch.bfloat16, (m, self.hq, self.d), "out")
        self._bind()
        check(self._lib.sve_extend_attn(self.ctx, slot, layer, _ptr(q), _ptr(new_k),
                                        _ptr(new_v), m, _ptr(out)), self.ctx)
        return out

    def extend_attn_batched(self, slots, ms, layer: int, q: torch.Tensor, new_k: torch.Tensor,
                            new_v: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """extend_attn over several slots in one launch; rows packed slot after slot."""
        slots = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
        ms = np.ascontiguousarray(np.asarray(ms, dtype=np.int32))
        total = int(ms.sum())
        _need(q, torch.bfloat16, (total, self.hq, self.d), "q")
        _need(new_k, torch.bfloat16, (total, self.hkv, self.d), "new_k")
        _need(new_v, torch.bfloat16, (total, self.hkv, self.d), "new_v")
        if out is None:
            out = torch.empty_like(q)
        _need(out, torch.bfloat16, (total, self.hq, self.d), "out")
        self._bind()
        check(self._lib.sve_extend_attn_batched(
            self.ctx, len(slots), slots.ctypes.data_as(C.c_void_p),
            ms.ctypes.data_as(C.c_void_p), layer, _ptr(q), _ptr(new_k), _ptr(new_v),
            _ptr(out)), self.ctx)
        return out

    def extend_attn_questions(self, slot: int, layer: int, ms, q: torch.Tensor,
                              new_k: torch.Tensor, new_v: torch.Tensor,
                              out: torch.Tensor | None = None) -> torch.Tensor:
        """Several questions on the slot's resident prefix in one launch (rows
        packed question after question); each sees the prefix and its own
        rows; nothing is appended."""
        ms = np.ascontiguousarray(np.asarray(ms, dtype=np.int32))
        total = int(ms.sum())
        _need(q, torch.bfloat16, (total, self.hq, self.d), "q")
        _need(new_k, torch.bfloat16, (total, self.hkv, self.d), "new_k")
        _need(new_v, torch.bfloat16, (total, self.hkv, self.d), "new_v")
        if out is None:
            out = torch.empty_like(q)
        _need(out, torch.bfloat16, (total, self.hq, self.d), "out")
        self._bind()
        check(self._lib.sve_extend_attn_questions(
            self.ctx, slot, layer, len(ms), ms.ctypes.data_as(C.c_void_p), _ptr(q), _ptr(new_k),
            _ptr(new_v), _ptr(out)), self.ctx)
        return out

    def timing_start(self, n_calls: int) -> None:
        """Record HIP events around the kernels of the next n_calls extend calls."""
        check(self._lib.sve_timing_start(self.ctx, int(n_calls)), self.ctx)

    def timing_read(self) -> dict:
        """Summed kernel durations (ms) of the timed extend calls; ends timing."""
        a, b, c, n = C.c_float(), C.c_float(), C.c_float(), C.c_int32()
        check(self._lib.sve_timing_read(self.ctx, C.byref(a), C.byref(b), C.byref(c), C.byref(n)),
              self.ctx)
        return {"append_ms": a.value, "attn_ms": b.value, "combine_ms": c.value, "calls": n.value}

    def kv_read(self, slot: int, layer: int, start: int, length: int):
        """Cached K and V rows [start, start+length) as bf16 [length][Hkv][D]."""
        k = torch.empty((length, self.hkv, self.d), dtype=torch.bfloat16, device=self.arena.device)
        v = torch.empty_like(k)
        self._bind()
        check(self._lib.sve_kv_read(self.ctx, slot, layer, start, length, _ptr(k), _ptr(v)),
              self.ctx)
        return k, v


def w4_packed_bytes(n: int, k: int) -> int:
    return int(_lib.load().sve_w4_packed_bytes(n, k))


def w4_pack(w: torch.Tensor, scales: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Device layout of an int4 group-32 weight (w uint8 [N][K/2], scales
    fp16 [N][K/32])."""
    lib = _lib.load()
    _need(w, torch.uint8, (n, k // 2), "w")
    _need(scales, torch.float16, (n, k // 32), "scales")
    nbytes = lib.sve_w4_packed_bytes(n, k)
    if nbytes == 0:
        raise ValueError("need N >= 1 and K % 32 == 0")
    packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    check(lib.sve_w4_pack(_ptr(w), _ptr(scales), n, k, _ptr(packed), _stream()))
    return packed


def w4_dequant(packed: torch.Tensor, n: int, k: int) -> torch.Tensor:
    lib = _lib.load()
    _need(packed, torch.uint8, (lib.sve_w4_packed_bytes(n, k),), "packed")
    out = torch.empty((n, k), dtype=torch.float32, device=packed.device)
    check(lib.sve_w4_dequant(_ptr(packed), n, k, _ptr(out), _stream()))
    return out


def w4_gemv_m(x: torch.Tensor, packed: torch.Tensor, n: int, k: int,
              y: torch.Tensor | None = None) -> torch.Tensor:
    """y [m][N] fp32 = x [m][K] bf16 times the packed int4 weight."""
    lib = _lib.load()
    m = x.shape[0]
    _need(x, torch.bfloat16, (m, k), "x")
    _need(packed, torch.uint8, (lib.sve_w4_packed_bytes(n, k),), "packed")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, (m, n), "y")
    check(lib.sve_w4_gemv_m(_ptr(x), m, _ptr(packed), n, k, _ptr(y), _stream()))
    return y


def w4_gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    """Device workspace bytes w4_gemm needs for this shape (0: none)."""
    return int(_lib.load().sve_w4_gemm_workspace_bytes(m, n, k))


def w4_gemm(x: torch.Tensor, packed: torch.Tensor, n: int, k: int,
            y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y [m][N] fp32 = x [m][K] bf16 times the packed int4 weight, any m."""
    lib = _lib.load()
    m = x.shape[0]
    _need(x, torch.bfloat16, (m, k), "x")
    _need(packed, torch.uint8, (lib.sve_w4_packed_bytes(n, k),), "packed")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, (m, n), "y")
    if workspace is None:
        workspace = torch.empty(max(lib.sve_w4_gemm_workspace_bytes(m, n, k), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, torch.uint8, None, "workspace")
    check(lib.sve_w4_gemm(_ptr(x), m, _ptr(packed), n, k, _ptr(y), _ptr(workspace),
                          workspace.numel(), _stream()))
    return y


def w4_gemv_m_routed(x: torch.Tensor, expert_ids: torch.Tensor, packed_all: torch.Tensor,
                     n_experts: int, n: int, k: int, x_per_slot: bool = False,
                     y: torch.Tensor | None = None) -> torch.Tensor:
    """y [m][topk][N] fp32: each (row, expert slot) through its own expert."""
    lib = _lib.load()
    m, topk = expert_ids.shape
    _need(expert_ids, torch.int32, (m, topk), "expert_ids")
    _need(x, torch.bfloat16, (m, topk, k) if x_per_slot else (m, k), "x")
    _need(packed_all, torch.uint8, (n_experts * lib.sve_w4_packed_bytes(n, k),), "packed_all")
    if y is None:
        y = torch.empty((m, topk, n), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, (m, topk, n), "y")
    check(lib.sve_w4_gemv_m_routed(_ptr(x), int(bool(x_per_slot)), m, _ptr(expert_ids), topk,
                                   _ptr(packed_all), n_experts, n, k, _ptr(y), _stream()))
    return y


def ngram_draft(tokens, k: int, max_ngram: int = 3, min_ngram: int = 1) -> np.ndarray:
    """Prompt-lookup draft: the up to k tokens that followed the latest
    earlier occurrence of the history's longest repeated suffix (host)."""
    lib = _lib.load()
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    out = np.zeros(max(int(k), 1), dtype=np.int32)
    cnt = C.c_int32(0)
    check(lib.sve_ngram_draft(t.ctypes.data_as(C.c_void_p) if t.size else None, int(t.size),
                              int(k), int(max_ngram), int(min_ngram),
                              out.ctypes.data_as(C.c_void_p), C.byref(cnt)))
    return out[:cnt.value].copy()


def verify_workspace_bytes(m: int, vocab: int) -> int:
    """Device workspace bytes of verify_accept for m rows of `vocab` logits."""
    return int(_lib.load().sve_verify_workspace_bytes(m, vocab))


def verify_accept(logits: torch.Tensor, draft: torch.Tensor | None,
                  result: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Greedy acceptance of one verify step (asynchronous).

    logits: fp32 [m][V] (rows for the last accepted token and the k = m-1
    drafts); draft: int32 [m-1] (None when m == 1). Returns int32 [2 + m]:
    accepted drafts, next token, per-row argmax."""
    lib = _lib.load()
    m, vocab = logits.shape
    _need(logits, torch.float32, (m, vocab), "logits")
    if m > 1 or draft is not None:
        _need(draft, torch.int32, (m - 1,), "draft")
    ws_bytes = lib.sve_verify_workspace_bytes(m, vocab)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=logits.device)
    _need(workspace, torch.uint8, None, "workspace")
    if result is None:
        result = torch.empty(2 + m, dtype=torch.int32, device=logits.device)
    _need(result, torch.int32, (2 + m,), "result")
    check(lib.sve_verify_accept(_ptr(logits), m, vocab,
                                None if draft is None else _ptr(draft), _ptr(result),
                                _ptr(workspace), workspace.numel(), _stream()))
    return result


def verify_accept_noalloc(logits: torch.Tensor, draft: torch.Tensor | None,
                          result: torch.Tensor) -> torch.Tensor:
    """verify_accept without a workspace: the library keeps its partial
    results in a static per-GPU array and allocates nothing (the caller
    passes the result tensor). Calls that overlap on one GPU race."""
    lib = _lib.load()
    m, vocab = logits.shape
    _need(logits, torch.float32, (m, vocab), "logits")
    if m > 1 or draft is not None:
        _need(draft, torch.int32, (m - 1,), "draft")
    _need(result, torch.int32, (2 + m,), "result")
    check(lib.sve_verify_accept_noalloc(_ptr(logits), m, vocab,
                                        None if draft is None else _ptr(draft), _ptr(result),
                                        _stream()))
    return result


class SpecGate:
    """Rolling-acceptance gate of one request (host-side, libsve)."""

    def __init__(self, k: int, min_accept: float = 0.60, window: int = 8):
        self._g = _lib.SpecGate()
        check(_lib.load().sve_spec_gate_init(C.byref(self._g), k, float(min_accept), window))

    @property
    def k(self) -> int:
        return int(self._g.k)

    def step(self, accepted: int) -> int:
        """Record a verify step that kept `accepted` drafts; returns the next depth."""
        k_next = C.c_int32(0)
        check(_lib.load().sve_spec_gate_step(C.byref(self._g), int(accepted), C.byref(k_next)))
        return int(k_next.value)


def spec_break_even(a: float, b: float, k: int) -> float:
    """Break-even per-position acceptance of depth k under verify(m) = a + b*m."""
    return float(_lib.load().sve_spec_break_even(float(a), float(b), int(k)))


def probe_read(src: torch.Tensor, blocks: int, unroll: int = 4, threads: int = 256,
               mode: int = 0) -> torch.Tensor:
    """Streaming read of a device buffer (measurement probe). mode 0: plain
    loads, 1: nontemporal loads, 2: direct global-to-LDS loads, 3: the
    buffer (small) read over and over into LDS, 8 * unroll tiles of 32 KB per
    wave."""
    nbytes = src.numel() * src.element_size()
    sink = torch.empty(blocks * (1 if mode >= 2 else threads), dtype=torch.int32,
                       device=src.device)
    check(_lib.load().sve_probe_read(_ptr(src), nbytes, blocks, threads, unroll, mode, _ptr(sink),
                                     _stream()))
    return sink


def probe_compute(kind: int, blocks: int, iters: int, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Compute-ceiling probe (kind 0: bf16 MFMA 16x16x32, 1: bf16 MFMA
    32x32x16, 2: fp16 MFMA 16x16x32, 3: v_exp_f32, 4: LDS reads)."""
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    check(_lib.load().sve_probe_compute(kind, blocks, iters, _ptr(sink), _stream()))
    return sink


def probe_copy(src: torch.Tensor, dst: torch.Tensor, blocks: int) -> None:
    """Plain device copy (measurement probe and counter calibration)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst differ in size")
    check(_lib.load().sve_probe_copy(_ptr(src), _ptr(dst), n, blocks, _stream()))
