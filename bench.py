#!/usr/bin/env python3
"""Benchmark of the extend-prefill / m-row int4 GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
                    [--no-graph] [--layers L] [--calibrate] [--only SECTION]

Timed step (the headline): one turn of the agent-turn replay at turn 9 on a
7B-like attention layer (28 q / 4 KV heads, head_dim 128): the slot is cut
back to the 1668 cached tokens and selected for the 1922-token prompt (reuses
1668) before the timed region, then 254 new rows are extended in each of 128
attention layers (timed). 128
layers are rotated so that the 500 MB of KV read per step cannot sit in the
256 MB Infinity Cache. value = 254 new tokens per attention-layer pass / time
of one pass (step time / 128), the per-layer calls replayed from a captured
HIP graph.

The roofline object is for the step's dominant kernel, the extend attention
kernel: its duration is taken from HIP events that the library records on its
stream around that kernel in every call of the eager timed steps.

Also measured in the same run and reported beside it: the m-row int4 GEMV
(9B-like and 7B-like layers, m = 1..8, weights rotated over 8 copies, each
launch bracketed by HIP events, and a plain streaming read of the same
buffers as the achievable floor), the speculative-verify attention sweep
(2048 cached + m rows), the routed MoE GEMV (256 experts, top-8), and four
slots in rotation (batched extend). Inputs are seeded synthetic data with the
workloads' shapes, resident in HBM before timing starts. The CPU oracle is
timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import speculative_verify_extend_amd as sve  # noqa: E402
import synth  # noqa: E402

METRIC = "extend-prefill tok/s at 1668+254 ctx; m-row int4 GEMV GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
ROT_LAYERS = 128
# counter summary of the attention kernel at the headline workload, and the
# sources whose hash it records (a changed kernel makes its traffic stale)
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_mfma_replay7b_turn9_traffic.md")
ATTN_SOURCES = ["kernels_attn.hip", "common.h", "launch.h"]


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def f16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.float16).cuda()


class Timer:
    """HIP events on torch's current stream (the stream libsve launches on)."""

    def __init__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        torch.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


class Backlog:
    """A long streaming read queued ahead of eagerly launched calls, so that
    the host is ahead of the GPU and each bracketed kernel starts as soon as
    its predecessor ends."""

    def __init__(self, nbytes=1 << 30):
        self.buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")

    def __call__(self):
        sve.probe_read(self.buf, 1024, 1)


class HipEvents:
    """Timing events of the HIP runtime torch has loaded, created without a
    system-scope fence (hipEventDisableSystemFence): a default event writes
    back and invalidates caches when it is recorded, and that time would be
    counted as part of the bracketed kernel."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP status {rc}")

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._ok(self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS), "hipEventCreate")
            evs.append(e)
        return evs

    def record(self, e):
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._ok(self.hip.hipEventRecord(e, s), "hipEventRecord")

    def elapsed(self, a, b):
        f = ctypes.c_float()
        self._ok(self.hip.hipEventElapsedTime(ctypes.byref(f), a, b), "hipEventElapsedTime")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


_EVENTS = None


def bracket(calls, backlog):
    """Per-call durations (ms) from HIP events recorded on the current
    stream right before and after each call (one kernel each)."""
    global _EVENTS
    if _EVENTS is None:
        _EVENTS = HipEvents()
    ev = _EVENTS.create(2 * len(calls))
    torch.cuda.synchronize()
    backlog()
    for i, f in enumerate(calls):
        _EVENTS.record(ev[2 * i])
        f()
        _EVENTS.record(ev[2 * i + 1])
    torch.cuda.synchronize()
    out = [_EVENTS.elapsed(ev[2 * i], ev[2 * i + 1]) for i in range(len(calls))]
    _EVENTS.destroy(ev)
    return out


def graph_of(fn, reset=lambda: None, stream=None):
    """Capture fn's launches in a HIP graph (one eager run first; reset()
    restores the host state before each)."""
    reset()
    fn()
    torch.cuda.synchronize()
    reset()
    stream = stream or torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def attn_flops(P, m, hq, d):
    return 4 * d * hq * (m * P + m * (m + 1) // 2)


def attn_bytes(P, m, hq, hkv, d):
    return 2 * (P + m) * hkv * d * 2 + 2 * m * hq * d * 2 + 4 * m * hkv * d * 2


def exp_count(P, m, hq):
    """Exponentials of an extend: one per visible (row, head, key) pair."""
    return hq * (m * P + m * (m + 1) // 2)


def gemv_bytes(m, n, k):
    return n * (k // 2) + n * (k // 32) * 2 + 2 * m * k + 4 * m * n


def fit(ms, ts):
    m = np.asarray(ms, float)
    t = np.asarray(ts, float)
    b = ((m - m.mean()) * (t - t.mean())).sum() / ((m - m.mean()) ** 2).sum()
    a = t.mean() - b * m.mean()
    return float(a), float(b)


def attn_source_hash():
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "speculative_verify_extend_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_summary():
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]+)`", text, flags=re.M))
    if fields.get("source_sha256") != attn_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# headline: replay turn 9
# ---------------------------------------------------------------------------

class Replay:
    def __init__(self, layers=ROT_LAYERS):
        wl = synth.WORKLOADS["replay7b"]
        self.hq, self.hkv, self.d = wl["hq"], wl["hkv"], wl["d"]
        self.P, self.n = 1668, 1922
        self.m = self.n - self.P
        self.layers = layers
        prompts = synth.replay_prompt(wl["seed"], wl["prompt_lengths"])
        self.p_prev = prompts[7]   # turn 8's prompt: 1668 tokens
        self.p_turn = prompts[8]   # turn 9's prompt: 1922 tokens
        assert len(self.p_prev) == self.P and len(self.p_turn) == self.n
        self.st = sve.KVSlots(4, layers, self.hq, self.hkv, self.d, 2112, self.P)
        # prefix rows (shared by all layers' caches: same values, distinct memory)
        c = synth.attention_case(wl["seed"], self.hq, self.hkv, self.d, self.P, self.m)
        self.case = c
        slot, r = self.st.kv_slot_select(self.p_prev)
        assert (slot, r) == (0, 0)
        qp, kp, vp = bf16_dev(c["q_prefix"]), bf16_dev(c["k_prefix"]), bf16_dev(c["v_prefix"])
        for layer in range(layers):
            self.st.extend_attn(0, layer, qp, kp, vp)
        del qp, kp, vp
        # per-layer new rows and outputs (distinct buffers, rotated with the layer)
        g = synth.rng(wl["seed"], 77)
        self.q, self.k, self.v, self.out = [], [], [], []
        base = (bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"]))
        for layer in range(layers):
            if layer == 0:
                q, k, v = base
            else:
                q, k, v = (bf16_dev(a) for a in synth.attention_rows(g, self.m, self.hq, self.hkv, self.d))
            self.q.append(q)
            self.k.append(k)
            self.v.append(v)
            self.out.append(torch.empty_like(q))
        torch.cuda.synchronize()

    def select(self):
        self.st.kv_truncate(0, self.P)
        slot, r = self.st.kv_slot_select(self.p_turn)
        assert (slot, r) == (0, self.P), (slot, r)

    def extend_all(self):
        for layer in range(self.layers):
            self.st.extend_attn(0, layer, self.q[layer], self.k[layer], self.v[layer], self.out[layer])

    def step(self, backlog=None):
        self.select()
        if backlog:
            backlog()
        self.extend_all()

    def capture(self):
        """Capture the per-layer extend calls of one step in a HIP graph
        (torch's graph capture records the library's launches on the capture
        stream). Replays repeat exactly these kernels: the step's KV rows are
        rewritten in place, so a replay after truncate + select is one turn."""
        self.select()
        stream = torch.cuda.Stream()
        self.graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph, stream=stream):
            self.extend_all()
        torch.cuda.synchronize()

    def step_graph(self):
        self.select()
        self.graph.replay()


def replay_turns(rp, passes=2, n_inputs=4, graph=True):
    """Every turn of the agent replay on the replay's store and rotated
    layers: turn t cuts the slot back to L_(t-1) resident rows (metadata
    only) and extends its m = L_t - L_(t-1) new rows in every layer. The
    slot's committed prompt is turn 9's, which starts with every earlier
    prompt, so no select is needed between turns. Per call: the kernel
    durations the library records with HIP events (eager calls); with
    `graph`, also the turn's calls captured in a HIP graph and replayed, on
    the library's own choice of kernel and on each many-row path forced. The
    new rows rotate over a few input buffers; the KV read per layer is the
    store's, distinct per layer."""
    wl = synth.WORKLOADS["replay7b"]
    lengths = list(wl["prompt_lengths"])[:9]  # turn 10's length is an extrapolation
    starts = [0] + lengths[:-1]
    mmax = max(b - a for a, b in zip(starts, lengths))
    g = synth.rng(wl["seed"], 91)
    ins = [tuple(bf16_dev(a) for a in synth.attention_rows(g, mmax, rp.hq, rp.hkv, rp.d))
           for _ in range(n_inputs)]
    out = torch.empty((mmax, rp.hq, rp.d), dtype=torch.bfloat16, device="cuda")
    res = {}
    for t, (P, n) in enumerate(zip(starts, lengths), start=1):
        m = n - P

        def one_pass():
            rp.st.kv_truncate(0, P)
            for layer in range(rp.layers):
                q, k, v = ins[layer % n_inputs]
                rp.st.extend_attn(0, layer, q[:m], k[:m], v[:m], out[:m])

        one_pass()
        torch.cuda.synchronize()
        rp.st.timing_start(passes * rp.layers)
        for _ in range(passes):
            one_pass()
        kt = rp.st.timing_read()
        c = kt["calls"]
        attn = kt["attn_ms"] / c * 1e3
        call = (kt["attn_ms"] + kt["append_ms"] + kt["combine_ms"]) / c * 1e3
        tf = attn_flops(P, m, rp.hq, rp.d) / (attn * 1e-6) / 1e12
        res[t] = {"cached": P, "new": m, "attn_us": r2(attn), "call_kernels_us": r2(call),
                  "tok_per_s": round(m / (call * 1e-6), 1), "attn_TFLOPs": round(tf, 1),
                  "attn_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        if graph:
            # the same pass captured in a HIP graph and replayed, on the
            # library's own choice of kernel and on each many-row path forced
            for name, path in (("graph_us_per_layer", None), ("graph_us_split_path", "mfma"),
                               ("graph_us_row_tile_path", "rows")):
                res[t][name] = r2(turn_graph_us(rp, P, m, ins, out, path))
            one_pass()  # (the turn's rows resident again for the next turn's cut)
            torch.cuda.synchronize()
    return res


def turn_graph_us(rp, P, m, ins, out, path, reps=5):
    """Per-layer time of one replay turn's extend calls (every layer) captured
    in a HIP graph, best of `reps` replays; `path` forces SVE_ATTN_PATH."""
    old = os.environ.get("SVE_ATTN_PATH")
    if path:
        os.environ["SVE_ATTN_PATH"] = path
    else:
        os.environ.pop("SVE_ATTN_PATH", None)
    try:
        n_in = len(ins)
        stream = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        rp.st.kv_truncate(0, P)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for layer in range(rp.layers):
                q, k, v = ins[layer % n_in]
                rp.st.extend_attn(0, layer, q[:m], k[:m], v[:m], out[:m])
        torch.cuda.synchronize()
        best = math.inf
        for _ in range(reps):
            rp.st.kv_truncate(0, P)
            with Timer() as tm:
                g.replay()
            best = min(best, tm.ms / rp.layers * 1e3)
        del g
        rp.st.kv_truncate(0, P)
        return best
    finally:
        if old is None:
            os.environ.pop("SVE_ATTN_PATH", None)
        else:
            os.environ["SVE_ATTN_PATH"] = old


def replay_turns_alone(layers):
    """replay_turns on a store of its own, eager calls only (for counter and
    trace runs)."""
    rp = Replay(layers)
    rp.select()
    return replay_turns(rp, graph=False)


# ---------------------------------------------------------------------------
# measured HBM ceilings
# ---------------------------------------------------------------------------

# read-probe launch shapes (mode, threads, blocks, loads in flight) that came
# out best over a sweep of 152 shapes at 9-57 MB and 1 GiB on this chip
# (mode 0: plain loads, 1: nontemporal loads, 2: direct global-to-LDS loads)
READ_SHAPES = [(2, 1024, 512, 1), (2, 512, 256, 4), (2, 256, 512, 4), (2, 1024, 256, 8),
               (0, 512, 1024, 8), (1, 512, 512, 2), (1, 1024, 256, 2), (1, 256, 256, 16)]


def read_ceiling_us(bufs, backlog, shapes=READ_SHAPES, reps=2):
    """Fastest plain read of same-sized buffers (rotated): the median
    per-launch time (ms) of the best launch shape. At most 8 launches per
    event bracket, so the host stays ahead of the GPU."""
    lib, st = sve.load_library(), sve._stream()
    best = math.inf
    for mode, threads, blocks, unroll in shapes:
        nb = bufs[0].numel() * bufs[0].element_size()
        if mode == 2 and (nb % 1024 or nb >= (1 << 31)):
            continue
        sink = torch.empty(blocks * threads, dtype=torch.int32, device="cuda")
        calls = [lambda p=sve._ptr(b), sp=sve._ptr(sink): lib.sve_probe_read(
            p, nb, blocks, threads, unroll, mode, sp, st) for b in bufs]
        d = []
        for _ in range(reps):
            for i in range(0, len(calls), 8):
                d += bracket(calls[i:i + 8], backlog)
        best = min(best, float(np.median(d)))
    return best


def ceilings(backlog):
    """Measured ceilings of this chip beside the published peaks: HBM read
    (1 GiB, best launch shape) and copy, bf16 / fp16 MFMA issue rate,
    v_exp_f32 throughput and LDS read bandwidth (kernels in libsve's probe
    file, HIP events per launch)."""
    buf = backlog.buf
    read = read_ceiling_us([buf] * 3, backlog, reps=1)
    half = buf.numel() // 2
    src, dst = buf[:half], buf[half:]
    copy = min(bracket([lambda: sve.probe_copy(src, dst, 2048)] * 3, backlog))
    out = {"hbm_read_GBps": round(buf.numel() / (read * 1e-3) / 1e9, 1),
           "hbm_copy_GBps": round(2 * half / (copy * 1e-3) / 1e9, 1)}
    blocks, iters = 2048, 2000
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    waves = blocks * 4
    per_wave = {0: ("mfma_bf16_16x16x32_TFLOPs", 8 * 16384 / 1e12),
                1: ("mfma_bf16_32x32x16_TFLOPs", 8 * 32768 / 1e12),
                2: ("mfma_f16_16x16x32_TFLOPs", 8 * 16384 / 1e12),
                3: ("v_exp_f32_T_per_s", 64 * 64 / 1e12),
                4: ("lds_read_TBps", 8 * 1024 / 1e12)}
    for kind, (name, per) in per_wave.items():
        sve.probe_compute(kind, blocks, iters, sink)
        ms = min(bracket([lambda k=kind: sve.probe_compute(k, blocks, iters, sink)] * 3, backlog))
        out[name] = round(per * waves * iters / (ms * 1e-3), 2)
    # one CU filling LDS from L2: a 1 MB region read over and over, one
    # 4-wave workgroup per CU, 128 tiles of 32 KB per wave
    region = buf[:1 << 20]
    sve.probe_read(region, 256, unroll=16, threads=256, mode=3)
    ms = min(bracket([lambda: sve.probe_read(region, 256, unroll=16, threads=256, mode=3)] * 3,
                     backlog))
    out["l2_lds_fill_GBps_per_CU"] = round(4 * 128 * 32768 / (ms * 1e-3) / 1e9, 1)
    out["what"] = ("HBM: streaming read of 1 GiB (best of the read-probe launch shapes) and copy "
                   "of 512 MiB; compute: 2048 workgroups x 4 waves x 2000 iterations of 8 matrix "
                   "products, 64 exponentials or 8 wave-wide 16-byte LDS reads; L2 to LDS: a "
                   "1 MB region read into LDS over and over by 256 workgroups of 4 waves (direct "
                   "loads, 32 KB in flight per wave); HIP events")
    return out


# ---------------------------------------------------------------------------
# GEMV sweep
# ---------------------------------------------------------------------------

def gemv_sweep(shapes, backlog, copies=8, m_values=range(1, 9), seed=3, reps=3):
    """Per m: each matrix's launches bracketed by HIP events (median over the
    rotated copies and repeats), the layer's sum, and a plain read of the
    same packed buffers (the floor a weight-streaming kernel can reach)."""
    g = synth.rng(seed, 55)
    mats = []
    for (n, k) in shapes:
        w, s = synth.w4_weights(g, n, k)
        wd, sd = torch.from_numpy(w).cuda(), f16_dev(s)
        packs = [sve.w4_pack(wd, sd, n, k) for _ in range(copies)]
        mats.append((n, k, packs))
        del wd, sd
    kmax = max(k for _, k in shapes)
    xs = [bf16_dev(synth.normal_bf16(g, (8, kmax))) for _ in range(copies)]
    floors = {(n, k): read_ceiling_us(packs, backlog) for (n, k, packs) in mats}
    res = {}
    for m in m_values:
        per = {}
        for (n, k, packs) in mats:
            xk = [x[:m, :k].contiguous() for x in xs]
            ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _ in range(copies)]
            calls = [lambda c=c: sve.w4_gemv_m(xk[c], packs[c], n, k, ys[c]) for c in range(copies)]
            for f in calls:
                f()
            d = []
            for _ in range(reps):
                d += bracket(calls, backlog)
            t = float(np.median(d))
            nb = gemv_bytes(m, n, k)
            per[f"{n}x{k}"] = dict(us=t * 1e3, GBps=nb / (t * 1e-3) / 1e9, bytes=nb,
                                   floor_us=floors[(n, k)] * 1e3)
        us = sum(v["us"] for v in per.values())
        nbytes = sum(v["bytes"] for v in per.values())
        floor = sum(v["floor_us"] for v in per.values())
        res[m] = dict(us=us, GBps=nbytes / (us * 1e-6) / 1e9, bytes=nbytes, floor_us=floor,
                      per_matrix=per)
    return res


def prefill_gemm_sweep(shapes, backlog, m_values=(254, 134), copies=4, seed=5, reps=3):
    """Many-row int4 GEMM (a prefill's projections): per m, each matrix's
    calls (fp16 packing of x, the product, the k-split sum when used)
    bracketed by HIP events, median over rotated weight copies and repeats."""
    g = synth.rng(seed, 77)
    mats = []
    for (n, k) in shapes:
        w, s = synth.w4_weights(g, n, k)
        wd, sd = torch.from_numpy(w).cuda(), f16_dev(s)
        mats.append((n, k, [sve.w4_pack(wd, sd, n, k) for _ in range(copies)]))
        del wd, sd
    kmax = max(k for _, k in shapes)
    res = {}
    for m in m_values:
        x = bf16_dev(synth.normal_bf16(g, (m, kmax)))
        per = {}
        for (n, k, packs) in mats:
            xk = x[:, :k].contiguous()
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            ws = torch.empty(sve.w4_gemm_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
            calls = [lambda c=c: sve.w4_gemm(xk, packs[c], n, k, y, ws) for c in range(copies)]
            for f in calls:
                f()
            d = []
            for _ in range(reps):
                d += bracket(calls, backlog)
            t = float(np.median(d))
            fl = 2 * m * n * k
            per[f"{n}x{k}"] = dict(us=t * 1e3, TFLOPs=fl / (t * 1e-3) / 1e12, flops=fl)
        us = sum(v["us"] for v in per.values())
        fl = sum(v["flops"] for v in per.values())
        res[m] = dict(us=us, TFLOPs=fl / (us * 1e-6) / 1e12, flops=fl, per_matrix=per)
    return res


def questions_sweep(backlog, layers=64, prefix=1250, ms=(30, 24, 36, 27), reps=3):
    """Several questions about one state (4B-like heads): one questions call
    per layer against the previous way, one extend per question with the
    slot cut back to the state after each. HIP events per layer; the state
    rotates over `layers` layers (5.1 MB of KV each)."""
    hq, hkv, d = 32, 8, 128
    total = int(sum(ms))
    st = sve.KVSlots(1, layers, hq, hkv, d, prefix + 128, max(prefix, total))
    st.kv_slot_select(np.arange(prefix + max(ms), dtype=np.int32))
    c = synth.attention_case(71, hq, hkv, d, prefix, total)
    qp, kp, vp = bf16_dev(c["q_prefix"]), bf16_dev(c["k_prefix"]), bf16_dev(c["v_prefix"])
    for layer in range(layers):
        st.extend_attn(0, layer, qp, kp, vp)
    del qp, kp, vp
    q, k, v = bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"])
    out = torch.empty_like(q)
    starts = np.concatenate([[0], np.cumsum(ms)[:-1]]).tolist()
    parts = [(q[s0:s0 + m], k[s0:s0 + m], v[s0:s0 + m], out[s0:s0 + m]) for s0, m in zip(starts, ms)]

    def together(layer):
        st.extend_attn_questions(0, layer, list(ms), q, k, v, out)

    def separate(layer):
        for (qq, kk, vv, oo) in parts:
            st.extend_attn(0, layer, qq, kk, vv, oo)
            st.kv_truncate(0, prefix)

    res = {}
    for name, fn in (("one_call", together), ("per_question", separate)):
        calls = [lambda L=L: fn(L) for L in range(layers)]
        for f in calls[:4]:
            f()
        d = []
        for _ in range(reps):
            d += bracket(calls, backlog)
        res[name] = float(np.median(d)) * 1e3
    res["speedup"] = res["per_question"] / res["one_call"]
    return res


# ---------------------------------------------------------------------------
# verify attention sweep (9B-like, 2048 cached)
# ---------------------------------------------------------------------------

def verify_sweep(backlog, layers=ROT_LAYERS, reps=3, graphs=True):
    wl = synth.WORKLOADS["verify9b"]
    hq, hkv, d, P = wl["hq"], wl["hkv"], wl["d"], wl["context"]
    st = sve.KVSlots(1, layers, hq, hkv, d, P + 64, P)
    st.kv_slot_select(np.arange(P + 8, dtype=np.int32))
    c = synth.attention_case(wl["seed"], hq, hkv, d, P, 8)
    qp, kp, vp = bf16_dev(c["q_prefix"]), bf16_dev(c["k_prefix"]), bf16_dev(c["v_prefix"])
    for layer in range(layers):
        st.extend_attn(0, layer, qp, kp, vp)
    del qp, kp, vp
    q, k, v = bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"])
    res = {}
    for m in range(1, 9):
        qm, km, vm = q[:m].contiguous(), k[:m].contiguous(), v[:m].contiguous()
        out = torch.empty_like(qm)

        def run():
            for layer in range(layers):
                st.extend_attn(0, layer, qm, km, vm, out)
        # kernel durations from the library's events (eager)
        st.kv_truncate(0, P)
        st.timing_start(layers)
        torch.cuda.synchronize()
        backlog()
        run()
        kt = st.timing_read()
        r = dict(attn_kernel_us=kt["attn_ms"] / kt["calls"] * 1e3,
                 append_kernel_us=kt["append_ms"] / kt["calls"] * 1e3,
                 combine_kernel_us=kt["combine_ms"] / kt["calls"] * 1e3)
        if graphs:
            gr = graph_of(run, reset=lambda: st.kv_truncate(0, P))
            best = math.inf
            for _ in range(reps):
                st.kv_truncate(0, P)
                with Timer() as t:
                    gr.replay()
                best = min(best, t.ms / layers)
            r["call_us"] = best * 1e3
            del gr
        st.kv_truncate(0, P)
        r["GBps_attn_kernel"] = attn_bytes(P, m, hq, hkv, d) / (r["attn_kernel_us"] * 1e-6) / 1e9
        res[m] = r
    st.close()
    return res


def verify_step_graph(layers=32, copies=8, reps=3):
    """One 9B-like layer of a verify step as a serving loop runs it: per
    layer the QKV GEMV, the attention call over 2048 cached + m rows, then the
    O, gate|up and down GEMVs, all layers captured in one HIP graph (each
    layer its own KV and one of `copies` rotated weight copies), per-layer
    time of the replay, best of `reps`. The GEMVs read fixed activation
    buffers (the step's data flow is not modelled, only its launches and
    bytes)."""
    wl = synth.WORKLOADS["verify9b"]
    hq, hkv, d, P = wl["hq"], wl["hkv"], wl["d"], wl["context"]
    st = sve.KVSlots(1, layers, hq, hkv, d, P + 64, P)
    st.kv_slot_select(np.arange(P + 8, dtype=np.int32))
    c = synth.attention_case(wl["seed"], hq, hkv, d, P, 8)
    qp, kp, vp = bf16_dev(c["q_prefix"]), bf16_dev(c["k_prefix"]), bf16_dev(c["v_prefix"])
    for layer in range(layers):
        st.extend_attn(0, layer, qp, kp, vp)
    del qp, kp, vp
    q, k, v = bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"])
    g = synth.rng(3, 56)
    shapes = synth.layer_gemv_shapes(4096, 12288, 32, 8, 128)
    mats = []
    for (n, kk) in shapes:
        w, sc = synth.w4_weights(g, n, kk)
        wd, sd = torch.from_numpy(w).cuda(), f16_dev(sc)
        mats.append((n, kk, [sve.w4_pack(wd, sd, n, kk) for _ in range(copies)]))
        del wd, sd
    kmax = max(kk for _, kk in shapes)
    x = bf16_dev(synth.normal_bf16(g, (8, kmax)))
    res = {}
    for m in range(1, 9):
        qm, km, vm = q[:m].contiguous(), k[:m].contiguous(), v[:m].contiguous()
        out = torch.empty_like(qm)
        xs = {kk: x[:m, :kk].contiguous() for _, kk, _ in mats}
        ys = {n: torch.empty((m, n), dtype=torch.float32, device="cuda") for n, _, _ in mats}

        def gemv(i, layer):
            n, kk, packs = mats[i]
            sve.w4_gemv_m(xs[kk], packs[layer % copies], n, kk, ys[n])

        def run():
            for layer in range(layers):
                gemv(0, layer)
                st.extend_attn(0, layer, qm, km, vm, out)
                for i in (1, 2, 3):
                    gemv(i, layer)

        gr = graph_of(run, reset=lambda: [st.kv_truncate(0, P)])
        best = math.inf
        for _ in range(reps):
            st.kv_truncate(0, P)
            with Timer() as t:
                gr.replay()
            best = min(best, t.ms / layers * 1e3)
        del gr
        res[m] = best
    st.close()
    return res


# ---------------------------------------------------------------------------
# verify acceptance (greedy argmax over a Qwen-family vocabulary)
# ---------------------------------------------------------------------------

def verify_accept_sweep(backlog, copies=8, reps=3):
    """Per m = k+1: time of one sve_verify_accept call (both kernels, HIP
    events around the call) on fp32 logits [m][151936], rotated over
    `copies` buffers; GB/s on the m*V*4 logit bytes."""
    vocab = synth.VERIFY_VOCAB
    res = {}
    for m in range(1, 9):
        cases = [synth.verify_case(90 + i, m, vocab, (m - 1) // 2) for i in range(copies)]
        lg = [torch.from_numpy(c[0]).cuda() for c in cases]
        dr = [torch.from_numpy(c[1]).cuda() if m > 1 else None for c in cases]
        ws = torch.empty(sve.verify_workspace_bytes(m, vocab), dtype=torch.uint8, device="cuda")
        out = [torch.empty(2 + m, dtype=torch.int32, device="cuda") for _ in range(copies)]
        calls = [lambda i=i: sve.verify_accept(lg[i], dr[i], out[i], ws) for i in range(copies)]
        d = []
        for _ in range(reps):
            d += bracket(calls, backlog)
        us = float(np.median(d)) * 1e3
        res[m] = {"us": us, "GBps": m * vocab * 4 / (us * 1e-6) / 1e9,
                  "accepted": int(out[0][0].item())}
        del lg, dr, ws, out
    return res


# ---------------------------------------------------------------------------
# MoE routed GEMV (35B-A3B-like)
# ---------------------------------------------------------------------------

def moe_sweep(backlog, n_routings=16, sets=2):
    wl = synth.WORKLOADS["moe35b"]
    E, hid, f, topk = wl["n_experts"], wl["hidden"], wl["expert_ffn"], wl["topk"]
    n1, k1, n2, k2 = 2 * f, hid, hid, f
    g = synth.rng(wl["seed"], 66)
    eb1 = sve.w4_packed_bytes(n1, k1)
    eb2 = sve.w4_packed_bytes(n2, k2)
    # one random expert matrix pair packed, replicated into every expert slot
    w1, s1 = synth.w4_weights(g, n1, k1)
    w2, s2 = synth.w4_weights(g, n2, k2)
    p1 = sve.w4_pack(torch.from_numpy(w1).cuda(), f16_dev(s1), n1, k1)
    p2 = sve.w4_pack(torch.from_numpy(w2).cuda(), f16_dev(s2), n2, k2)
    W1 = [p1.repeat(E) for _ in range(sets)]
    W2 = [p2.repeat(E) for _ in range(sets)]
    res = {}
    for m in range(1, 9):
        routs = [synth.routing_topk(g, m, E, topk)[0] for _ in range(n_routings)]
        ids = [torch.from_numpy(r).cuda() for r in routs]
        union = [len(set(r.ravel().tolist())) for r in routs]
        x = bf16_dev(synth.normal_bf16(g, (m, k1)))
        h = bf16_dev(synth.normal_bf16(g, (m, topk, k2)))
        y1 = torch.empty((m, topk, n1), dtype=torch.float32, device="cuda")
        y2 = torch.empty((m, topk, n2), dtype=torch.float32, device="cuda")
        up = [lambda i=i: sve.w4_gemv_m_routed(x, ids[i], W1[i % sets], E, n1, k1, False, y1)
              for i in range(n_routings)]
        down = [lambda i=i: sve.w4_gemv_m_routed(h, ids[i], W2[i % sets], E, n2, k2, True, y2)
                for i in range(n_routings)]
        for fn in up + down:
            fn()
        tu = bracket(up, backlog)
        td = bracket(down, backlog)
        us = (sum(tu) + sum(td)) / n_routings * 1e3
        ub = float(np.mean(union)) * (eb1 + eb2)
        res[m] = dict(us=us, up_us=float(np.median(tu)) * 1e3, down_us=float(np.median(td)) * 1e3,
                      union_experts=float(np.mean(union)), GBps=ub / (us * 1e-6) / 1e9)
    return res


# ---------------------------------------------------------------------------
# four slots in rotation (4B-like), batched extend
# ---------------------------------------------------------------------------

def slots_rotation(backlog):
    wl = synth.WORKLOADS["slots4b"]
    hq, hkv, d = wl["hq"], wl["hkv"], wl["d"]
    st = sve.KVSlots(4, 1, hq, hkv, d, 1024, 4 * 1024)
    order = synth.rotation_sessions(wl["seed"], 4, wl["turns"], wl["state_tokens"],
                                    wl["shared_start"], wl["question_min"], wl["question_max"])
    g = synth.rng(wl["seed"], 88)
    prefilled, kern, toks = [], [], 0
    for rnd in range(wl["turns"]):
        reqs = order[4 * rnd:4 * rnd + 4]
        sel = [st.kv_slot_select(p) for _, p in reqs]
        ms = [len(p) - r for (_, p), (_, r) in zip(reqs, sel)]
        prefilled.append(ms)
        total = sum(ms)
        q, k, v = (bf16_dev(a) for a in synth.attention_rows(g, total, hq, hkv, d))
        st.timing_start(1)
        torch.cuda.synchronize()
        backlog()
        st.extend_attn_batched([s for s, _ in sel], ms, 0, q, k, v)
        kt = st.timing_read()
        if rnd > 0:  # the first round fills the 800-token states
            kern.append(kt["append_ms"] + kt["attn_ms"] + kt["combine_ms"])
            toks += total
    st.close()
    return dict(prefilled_per_turn=prefilled,
                batched_tok_per_s=toks / (sum(kern) * 1e-3) if kern else None,
                kernel_ms_per_round=float(np.median(kern)) if kern else None)


# ---------------------------------------------------------------------------
# the tiny single-layer configuration (cache-resident: a correctness config)
# ---------------------------------------------------------------------------

def tiny_config(backlog, reps=20):
    """Tiny workload (4 q / 2 KV heads, D 64; 64 cached + 8 new rows; int4
    weight 1024 x 256): the extend and the GEMV at m = 1..8. Everything fits
    in the caches, so these are latencies, not a bandwidth measurement. Per
    call: `reps` calls captured in a HIP graph and replayed (GPU time with no
    host work between the kernels), and, for comparison, eager calls
    bracketed by HIP events, which at this size measure the Python call
    itself (the GPU finishes each call before the host has issued the next)."""
    wl = synth.WORKLOADS["tiny"]
    hq, hkv, d, P, m = wl["hq"], wl["hkv"], wl["d"], wl["prefix"], wl["m"]
    c = synth.attention_case(wl["seed"], hq, hkv, d, P, m)
    st = sve.KVSlots(1, 1, hq, hkv, d, 256, 64)
    st.kv_slot_select(np.arange(P + m, dtype=np.int32))
    st.extend_attn(0, 0, bf16_dev(c["q_prefix"]), bf16_dev(c["k_prefix"]), bf16_dev(c["v_prefix"]))
    q, k, v = bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"])
    out = torch.empty_like(q)

    def ext():
        st.kv_truncate(0, P)
        st.extend_attn(0, 0, q, k, v, out)

    def graph_us(fn):
        g = graph_of(lambda: [fn() for _ in range(reps)])
        best = math.inf
        for _ in range(5):
            with Timer() as t:
                g.replay()
            best = min(best, t.ms / reps * 1e3)
        del g
        return r2(best)
    ext_graph = graph_us(ext)
    ext_eager = float(np.median(bracket([ext] * reps, backlog))) * 1e3
    st.kv_truncate(0, P)
    n, kk = wl["gemv_n"], wl["gemv_k"]
    w, s = synth.w4_weights(synth.rng(wl["seed"], 7), n, kk)
    packed = sve.w4_pack(torch.from_numpy(w).cuda(), f16_dev(s), n, kk)
    x = bf16_dev(synth.normal_bf16(synth.rng(wl["seed"], 8), (8, kk)))
    gemv, gemv_eager = {}, {}
    for mm in range(1, 9):
        xm = x[:mm].contiguous()
        y = torch.empty((mm, n), dtype=torch.float32, device="cuda")
        call = lambda: sve.w4_gemv_m(xm, packed, n, kk, y)
        gemv[mm] = graph_us(call)
        gemv_eager[mm] = r2(float(np.median(bracket([call] * reps, backlog))) * 1e3)
    st.close()
    return {"workload": "tiny single layer: 4 q / 2 KV heads, D 64, 64 cached + 8 new rows; "
                        "int4 weight 1024 x 256 (group 32)",
            "cache_resident": True,
            "extend_us": ext_graph, "gemv_us_per_m": gemv,
            "timing": f"{reps} calls captured in a HIP graph, per call, best of 5 replays",
            "eager_call_us": {"extend": r2(ext_eager), "gemv_per_m": gemv_eager,
                              "note": "HIP events around each eager call from Python: at this "
                                      "size the GPU waits for the host, so this is the call "
                                      "overhead of the Python binding, not GPU time"},
            "note": "0.56 MFLOP and 49 KB of KV, 0.15 MB of weights: every operand is cache "
                    "resident, so the times are launch and latency bound"}


def gemv_content(backlog, m=8, copies=8, reps=3):
    """The GEMV's time does not depend on the values it multiplies (the
    weights are read once whatever the rows hold): the 9B-like layer at m
    rows with x ~ N(0,1), x = 0, x = +-1e4, and with every weight code 8
    (all-zero weights)."""
    g = synth.rng(3, 57)
    shapes = synth.layer_gemv_shapes(4096, 12288, 32, 8, 128)
    layer = {}
    for (n, k) in shapes:
        w, sc = synth.w4_weights(g, n, k)
        wd, sd = torch.from_numpy(w).cuda(), f16_dev(sc)
        eights = torch.full_like(wd, 0x88)
        layer[(n, k)] = ([sve.w4_pack(wd, sd, n, k) for _ in range(copies)],
                         [sve.w4_pack(eights, sd, n, k) for _ in range(copies)])
        del wd, sd, eights
    kmax = max(k for _, k in shapes)
    normal = synth.normal_bf16(g, (m, kmax))
    big = synth.f32_to_bf16_bits(np.where(g.random((m, kmax)) < 0.5, -1e4, 1e4).astype(np.float32))
    xs = {"normal": bf16_dev(normal), "zeros": torch.zeros((m, kmax), dtype=torch.bfloat16,
                                                           device="cuda"),
          "pm1e4": bf16_dev(big)}
    variants = [(name, xt, 0) for name, xt in xs.items()] + [("codes_all_8", xs["normal"], 1)]
    res = {}
    for name, xt, which in variants:
        tot = 0.0
        for (n, k), packs2 in layer.items():
            packs = packs2[which]
            xk = xt[:, :k].contiguous()
            ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _ in range(copies)]
            calls = [lambda c=c: sve.w4_gemv_m(xk, packs[c], n, k, ys[c]) for c in range(copies)]
            for f in calls:
                f()
            d = []
            for _ in range(reps):
                d += bracket(calls, backlog)
            tot += float(np.median(d)) * 1e3
        res[name] = r2(tot)
    vals = list(res.values())
    return {"workload": f"9B-like layer GEMVs at m = {m}, 8 rotated weight copies; layer time "
                        "(us) per content variant",
            "layer_us": res, "spread": round(max(vals) / min(vals) - 1.0, 4)}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_facts():
    """CPU model, the cores this process may run on, and numpy's BLAS
    (vendor, threads it uses)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    blas, threads = "unknown", affinity
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = "%s %s" % (infos[0].get("internal_api", "?"), infos[0].get("version", ""))
            threads = max(i.get("num_threads", 1) for i in infos)
    except Exception:
        pass
    return model, affinity, blas.strip(), threads


def cpu_baseline(case, P, budget_s=10.0):
    from oracle.attention import extend_attention
    model, affinity, blas, threads = cpu_facts()
    k_all = np.concatenate([case["k_prefix"], case["k"]])
    v_all = np.concatenate([case["v_prefix"], case["v"]])
    n, t0 = 0, time.perf_counter()
    while True:
        extend_attention(case["q"], k_all, v_all, P)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    m = case["q"].shape[0]
    return dict(value=m / dt, unit="tok/s", cores=int(threads), kind="oracle",
                sample=f"turn 9 of the replay, one 7B-like attention layer (1668 cached + {m} "
                       f"new rows, fp64 numpy), repeated {n}x over {budget_s:.0f} s",
                cpu_model=model, affinity_cores=int(affinity), blas=blas,
                cores_what="BLAS threads numpy used (the host's thread limit); affinity_cores "
                           "= CPUs this process may run on")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def r2(v):
    return round(float(v), 2)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the GEMV / GEMM / verify / MoE / slot sweeps")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the headline from eager launches only (for counter runs)")
    ap.add_argument("--layers", type=int, default=ROT_LAYERS)
    ap.add_argument("--only", choices=["gemv", "verify", "moe", "gemm", "accept", "ceilings",
                                       "tiny", "content", "turns", "verifystep"],
                    help="run one section alone and print its JSON (counter and trace runs)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the copy probe (256 MiB, three times): the known byte count "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is not sharded); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    sve.load_library()
    if args.calibrate:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            sve.probe_copy(src, dst, 4096)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": src.numel(), "launches": 3}))
        return

    if args.only:
        backlog = Backlog()
        for _ in range(200):
            backlog()
        torch.cuda.synchronize()
        sections = {
            "gemv": lambda: gemv_sweep(synth.layer_gemv_shapes(4096, 12288, 32, 8, 128), backlog,
                                       m_values=(1, 4, 8)),
            "verify": lambda: verify_sweep(backlog, layers=min(args.layers, ROT_LAYERS)),
            "verifystep": lambda: verify_step_graph(),
            "moe": lambda: moe_sweep(backlog),
            "gemm": lambda: prefill_gemm_sweep(synth.layer_gemv_shapes(3584, 18944, 28, 4, 128),
                                               backlog),
            "accept": lambda: verify_accept_sweep(backlog),
            "ceilings": lambda: ceilings(backlog),
            "tiny": lambda: tiny_config(backlog),
            "content": lambda: gemv_content(backlog),
            "turns": lambda: replay_turns_alone(args.layers),
        }
        log(args.only)
        print(json.dumps({args.only: sections[args.only]()}, default=float), flush=True)
        return

    backlog = Backlog()
    log("ceilings")
    for _ in range(200):  # clocks up before anything is timed
        backlog()
    torch.cuda.synchronize()
    ceil = ceilings(backlog)
    log("replay setup")
    rp = Replay(args.layers)
    for _ in range(args.warmup):
        rp.step()
    torch.cuda.synchronize()
    # eager steps: every layer's extend launched from Python; the library
    # records events around each call's kernels (the kernel durations of the
    # roofline). The events themselves cost GPU time between the kernels, so
    # the eager step time is taken again without them.
    rp.st.timing_start(args.steps * args.layers)
    ms_eager_timed = 0.0
    for _ in range(args.steps):
        rp.select()
        backlog()
        with Timer() as t:
            rp.extend_all()
        ms_eager_timed += t.ms
    kt = rp.st.timing_read()
    ms_eager_timed /= args.steps
    ms_eager = 0.0
    for _ in range(args.steps):
        rp.select()
        backlog()
        with Timer() as t:
            rp.extend_all()
        ms_eager += t.ms
    ms_eager /= args.steps
    calls = kt["calls"]
    attn_us = kt["attn_ms"] / calls * 1e3
    append_us = kt["append_ms"] / calls * 1e3
    combine_us = kt["combine_ms"] / calls * 1e3
    if args.no_graph:
        ms_step = ms_eager
    else:
        # graph: the same calls captured once and replayed
        rp.capture()
        for _ in range(args.warmup):
            rp.step_graph()
        torch.cuda.synchronize()
        ms_step = 0.0
        for _ in range(args.steps):
            rp.select()
            with Timer() as t:
                rp.graph.replay()
            ms_step += t.ms
        ms_step /= args.steps
    per_layer_s = ms_step * 1e-3 / args.layers
    value = rp.m / per_layer_s
    log(f"step {ms_step:.3f} ms (eager {ms_eager:.3f}), {per_layer_s * 1e6:.2f} us per layer; "
        f"kernels append {append_us:.2f} attn {attn_us:.2f} combine {combine_us:.2f} us")

    flops = attn_flops(rp.P, rp.m, rp.hq, rp.d)
    achieved = flops / (attn_us * 1e-6) / 1e12
    traffic = traffic_from_summary()
    roofline = {"bound": "mfma", "achieved": r2(achieved), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic,
                "kernel": "attn_mfma_kernel<128> (extend attention, 1668 cached + 254 rows, "
                          "28/4 heads, D 128)",
                "us_per_launch": r2(attn_us), "flops_per_launch": flops,
                "algorithmic_bytes_per_launch": attn_bytes(rp.P, rp.m, rp.hq, rp.hkv, rp.d),
                "timing": "HIP events recorded by the library on its stream around the kernel, "
                          f"averaged over {calls} eager calls",
                "other_kernels_us": {"kv_append": r2(append_us), "combine": r2(combine_us)},
                "measured_peak": ceil["mfma_bf16_16x16x32_TFLOPs"],
                "frac_of_measured": round(achieved / ceil["mfma_bf16_16x16x32_TFLOPs"], 4),
                "measured_peak_what": "v_mfma_f32_16x16x32_bf16 (the kernel's instruction) issued "
                                      "back to back on every SIMD (bench ceilings)",
                "exp_bound_us": r2(exp_count(rp.P, rp.m, rp.hq) / (ceil["v_exp_f32_T_per_s"] * 1e12)
                                   * 1e6)}
    if append_us == 0.0:
        roofline["other_kernels_us"]["kv_append"] = "none: the attention kernel appends the rows"

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tok/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "agent-turn replay turn 9: extend of 254 new rows over 1668 "
                                  "cached (the slot is cut back and selected before the timed "
                                  "region), 7B-like attention layer (28 q / 4 KV heads, D 128), "
                                  f"{args.layers} layers rotated, per-layer calls "
                                  + ("launched eagerly" if args.no_graph else
                                     "replayed from a captured HIP graph")
                                  + "; value = new tokens per layer pass",
                      "new_rows": rp.m, "cached": rp.P, "layers": args.layers},
           "roofline": roofline,
           "eager_launches": {"ms_per_step": round(ms_eager, 4),
                              "ms_per_step_with_kernel_events": round(ms_eager_timed, 4),
                              "what": "the same steps with every layer's call launched from "
                                      "Python (the host issues about 20 us per call); with the "
                                      "library's kernel events on, the events add GPU time "
                                      "between the kernels"}}

    if not args.no_extra:
        log("replay turns")
        out["replay_turns"] = {
            "workload": "every turn of the agent replay (7B-like attention, 28 q / 4 KV heads, "
                        "D 128; turn t: L_(t-1) cached + L_t - L_(t-1) new rows), "
                        f"{args.layers} layers rotated; per call: the summed kernel durations "
                        "from HIP events (eager calls), attention FLOPs / attention kernel time",
            "per_turn": replay_turns(rp)}
        out["ceilings"] = ceil
        log("gemv sweep")
        g9 = gemv_sweep(synth.layer_gemv_shapes(4096, 12288, 32, 8, 128), backlog)
        g7 = gemv_sweep(synth.layer_gemv_shapes(3584, 18944, 28, 4, 128), backlog, copies=6,
                        m_values=(1, 4, 8))
        a, b = fit(list(g9), [g9[m]["us"] for m in g9])
        worst = min(v["GBps"] for v in g9.values())
        out["gemv"] = {
            "workload": "9B-like layer (QKV 6144x4096, O 4096x4096, gate|up 24576x4096, "
                        "down 4096x12288), int4 group-32, 8 rotated copies; per-launch kernel "
                        "time from HIP events; layer = sum of the four launches",
            "roofline": {"bound": "hbm", "achieved": round(worst, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(worst / HBM_PEAK_GBS, 4),
                         "what": "worst m of 1..8, algorithmic bytes / summed kernel time",
                         "frac_of_measured": round(min(v["floor_us"] / v["us"] for v in g9.values()), 4),
                         "measured_what": "the same four launches' best plain read of the same "
                                          "packed buffers (per-size ceiling: launch, ramp and tail "
                                          "included) over the layer time, worst m"},
            "per_m": {m: {"us": r2(v["us"]), "GBps": round(v["GBps"], 1),
                          "frac": round(v["GBps"] / HBM_PEAK_GBS, 4),
                          "read_floor_us": r2(v["floor_us"]),
                          "per_matrix_us": {kk: r2(pv["us"]) for kk, pv in v["per_matrix"].items()}}
                      for m, v in g9.items()},
            "read_floor_per_matrix_us": {kk: r2(pv["floor_us"])
                                         for kk, pv in g9[1]["per_matrix"].items()},
            "fit_us": {"fixed": round(a, 3), "per_row": round(b, 3),
                       "per_row_over_fixed": round(b / a, 4)},
            "7b_layer_per_m": {m: {"us": r2(v["us"]), "GBps": round(v["GBps"], 1)}
                               for m, v in g7.items()},
        }
        log("prefill gemm")
        pg = prefill_gemm_sweep(synth.layer_gemv_shapes(3584, 18944, 28, 4, 128), backlog)
        best = pg[254]["TFLOPs"]
        out["prefill_gemm"] = {
            "workload": "7B-like layer projections (QKV 4608x3584, O 3584x3584, gate|up "
                        "37888x3584, down 3584x18944), int4 group-32 weights, m new rows "
                        "(254: the replay's turn 9; 134: its turns 2-8); each call = fp16 "
                        "packing of x + the product (+ the k-split sum), HIP events, 4 rotated "
                        "weight copies; layer = sum of the four calls",
            "roofline": {"bound": "mfma", "achieved": round(best, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(best / MFMA_BF16_PEAK_TFLOPS, 4),
                         "what": "m = 254, 2*m*N*K summed over the layer / summed call time; "
                                 "peak = dense fp16 (= bf16) MFMA"},
            "per_m": {m: {"us": r2(v["us"]), "TFLOPs": round(v["TFLOPs"], 1),
                          "new_tok_per_s_layer": round(m / (v["us"] * 1e-6), 1),
                          "per_matrix_us": {kk: r2(pv["us"]) for kk, pv in v["per_matrix"].items()}}
                      for m, v in pg.items()}}
        log("questions")
        qs = questions_sweep(backlog)
        out["questions"] = {
            "workload": "four questions (30, 24, 36, 27 rows) about one 1250-token state, 4B-like "
                        "heads (32 q / 8 KV, D 128), 64 layers rotated; per-layer time from HIP "
                        "events: one questions call (the state read once) against one extend per "
                        "question with the slot cut back after each",
            "one_call_us": r2(qs["one_call"]), "per_question_us": r2(qs["per_question"]),
            "speedup": round(qs["speedup"], 3)}
        log("verify sweep")
        vs = verify_sweep(backlog, layers=min(args.layers, ROT_LAYERS))
        a2, b2 = fit(list(vs), [vs[m]["attn_kernel_us"] for m in vs])
        out["verify_attention"] = {
            "workload": "9B-like attention (32 q / 8 KV heads, D 128), 2048 cached + m rows",
            "per_m": {m: {kk: r2(vv) for kk, vv in v.items()} for m, v in vs.items()},
            "fit_attn_kernel_us": {"fixed": round(a2, 3), "per_row": round(b2, 3)}}
        # the same sweep with each kernel path forced, as evidence for the
        # default path choice
        for path, rows in (("valu", "100000"), ("mfma", "1")):
            os.environ["SVE_MFMA_MIN_ROWS"] = rows
            vp = verify_sweep(backlog, layers=32, graphs=False)
            out["verify_attention"]["forced_" + path + "_attn_kernel_us"] = {
                m: r2(v["attn_kernel_us"]) for m, v in vp.items()}
        os.environ.pop("SVE_MFMA_MIN_ROWS", None)
        # one layer of a verify step: its four GEMVs plus the attention call
        # (thinkspread's verify(m) = fixed + per-row cost, per layer here)
        step = {m: g9[m]["us"] + vs[m]["call_us"] for m in range(1, 9)}
        a4, b4 = fit(list(step), list(step.values()))
        log("verify step graph")
        sg = verify_step_graph()
        a5, b5 = fit(list(sg), list(sg.values()))
        out["verify_step"] = {
            "workload": "one 9B-like layer of a verify step: the four int4 GEMVs (QKV, O, "
                        "gate|up, down) + the attention call over 2048 cached + m rows",
            "per_m_us": {m: r2(v) for m, v in step.items()},
            "fit_us": {"fixed": round(a4, 3), "per_row": round(b4, 3),
                       "per_row_over_fixed": round(b4 / a4, 4)},
            "timing": "sum of the GEMV launches' HIP-event times and the attention call's "
                      "graph-replay time",
            "graph": {"per_m_us": {m: r2(v) for m, v in sg.items()},
                      "fit_us": {"fixed": round(a5, 3), "per_row": round(b5, 3),
                                 "per_row_over_fixed": round(b5 / a5, 4)},
                      "timing": "32 layers, each QKV GEMV, attention, O, gate|up and down "
                                "captured in one HIP graph and replayed (rotated weight "
                                "copies), per layer"}}
        log("verify accept")
        va = verify_accept_sweep(backlog)
        out["verify_accept"] = {
            "workload": "greedy acceptance of m = k+1 verify rows over a 151936-id vocabulary "
                        "(fp32 logits, 8 rotated copies): per-row argmax + acceptance scan",
            "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "achieved": round(max(v["GBps"] for v in va.values()), 1),
                         "frac": round(max(v["GBps"] for v in va.values()) / HBM_PEAK_GBS, 4),
                         "what": "best m of 1..8, logit bytes / call time (two launches)"},
            "per_m": {m: {"us": r2(v["us"]), "GBps": round(v["GBps"], 1),
                          "accepted": v["accepted"]} for m, v in va.items()}}
        log("moe sweep")
        mo = moe_sweep(backlog)
        a3, b3 = fit(list(mo), [mo[m]["us"] for m in mo])
        out["moe"] = {
            "workload": "35B-A3B-like expert layer: 256 experts, W1 1024x2048, W2 2048x512, top-8",
            "per_m": {m: {"us": r2(v["us"]), "union_experts": r2(v["union_experts"]),
                          "GBps": round(v["GBps"], 1)} for m, v in mo.items()},
            "fit_us": {"fixed": round(a3, 3), "per_row": round(b3, 3)}}
        log("slots")
        out["slots"] = slots_rotation(backlog)
        log("tiny")
        out["tiny"] = tiny_config(backlog)
        log("gemv content")
        out["gemv_content"] = gemv_content(backlog)

    if not args.no_cpu:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline(rp.case, rp.P)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
