#!/usr/bin/env python3
"""Benchmark of the extend-prefill / m-row int4 GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

Timed step (the headline): one turn of the agent-turn replay at turn 9 on a
7B-like attention layer (28 q / 4 KV heads, head_dim 128): truncate the slot
back to the 1668 cached tokens, select the slot for the 1922-token prompt
(reuses 1668), then extend 254 new rows in each of 128 attention layers. 128
layers are rotated so that the 500 MB of KV read per step cannot sit in the
256 MB Infinity Cache. value = 254 new tokens per attention-layer pass / time
of one pass (step time / 128).

Also measured in the same run and reported beside it: the m-row int4 GEMV
(9B-like and 7B-like layers, m = 1..8, weights rotated over 8 copies), the
speculative-verify attention sweep (2048 cached + m rows), the routed MoE
GEMV (256 experts, top-8), and four slots in rotation (batched extend).
Inputs are seeded synthetic data with the workloads' shapes, resident in HBM
before timing starts. The CPU oracle is timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
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


def attn_flops(P, m, hq, d):
    return 4 * d * hq * (m * P + m * (m + 1) // 2)


def attn_bytes(P, m, hq, hkv, d):
    return 2 * (P + m) * hkv * d * 2 + 2 * m * hq * d * 2 + 4 * m * hkv * d * 2


def gemv_bytes(m, n, k):
    return n * (k // 2) + n * (k // 32) * 2 + 2 * m * k + 4 * m * n


def fit(ms, ts):
    m = np.asarray(ms, float)
    t = np.asarray(ts, float)
    b = ((m - m.mean()) * (t - t.mean())).sum() / ((m - m.mean()) ** 2).sum()
    a = t.mean() - b * m.mean()
    return float(a), float(b)


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

    def step(self):
        self.st.kv_truncate(0, self.P)
        slot, r = self.st.kv_slot_select(self.p_turn)
        assert (slot, r) == (0, self.P), (slot, r)
        for layer in range(self.layers):
            self.st.extend_attn(0, layer, self.q[layer], self.k[layer], self.v[layer], self.out[layer])

    def capture(self):
        """Capture the per-layer extend calls of one step in a HIP graph
        (torch's graph capture records the library's launches on the capture
        stream). Replays repeat exactly these kernels: the step's KV rows are
        rewritten in place, so a replay after truncate + select is one turn."""
        self.stream = torch.cuda.Stream()
        self.graph = torch.cuda.CUDAGraph()
        self.st.kv_truncate(0, self.P)
        self.st.kv_slot_select(self.p_turn)
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph, stream=self.stream):
            for layer in range(self.layers):
                self.st.extend_attn(0, layer, self.q[layer], self.k[layer], self.v[layer],
                                    self.out[layer])
        torch.cuda.synchronize()

    def step_graph(self):
        self.st.kv_truncate(0, self.P)
        slot, r = self.st.kv_slot_select(self.p_turn)
        assert (slot, r) == (0, self.P), (slot, r)
        self.graph.replay()

    def time_extend_graph(self, reps=5):
        best = math.inf
        for _ in range(reps):
            with Timer() as t:
                self.graph.replay()
            best = min(best, t.ms / self.layers)
        return best

    def time_extend_only(self, reps=3):
        """Average duration of one extend call (append + attention kernels)."""
        best = math.inf
        for _ in range(reps):
            self.st.kv_truncate(0, self.P)
            self.st.kv_slot_select(self.p_turn)
            with Timer() as t:
                for layer in range(self.layers):
                    self.st.extend_attn(0, layer, self.q[layer], self.k[layer], self.v[layer],
                                        self.out[layer])
            best = min(best, t.ms / self.layers)
        return best


# ---------------------------------------------------------------------------
# GEMV sweep
# ---------------------------------------------------------------------------

def gemv_sweep(shapes, copies=8, reps=5, m_values=range(1, 9), seed=3):
    g = synth.rng(seed, 55)
    mats = []
    for (n, k) in shapes:
        w, s = synth.w4_weights(g, n, k)
        wd, sd = torch.from_numpy(w).cuda(), f16_dev(s)
        packs = [sve.w4_pack(wd, sd, n, k) for _ in range(copies)]
        mats.append((n, k, packs))
        del wd, sd
    kmax = max(k for _, k in shapes)
    nmax = max(n for n, _ in shapes)
    xs = [bf16_dev(synth.normal_bf16(g, (8, kmax))) for _ in range(copies)]
    ys = [torch.empty((8, nmax), dtype=torch.float32, device="cuda") for _ in range(copies)]
    res = {}
    for m in m_values:
        # inputs and outputs per copy, prepared before timing
        xsl = {}
        for c in range(copies):
            for (n, k, _) in mats:
                xsl[(c, k)] = xs[c][:m, :k].contiguous()
        ysl = {}
        for c in range(copies):
            for (n, k, _) in mats:
                ysl[(c, n)] = torch.empty((m, n), dtype=torch.float32, device="cuda")

        def run2():
            for c in range(copies):
                for (n, k, packs) in mats:
                    sve.w4_gemv_m(xsl[(c, k)], packs[c], n, k, ysl[(c, n)])
        run2()
        best = math.inf
        for _ in range(reps):
            with Timer() as t:
                run2()
            best = min(best, t.ms / copies)
        nbytes = sum(gemv_bytes(m, n, k) for (n, k, _) in mats)
        res[m] = dict(us=best * 1e3, GBps=nbytes / (best * 1e-3) / 1e9, bytes=nbytes)
    return res


# ---------------------------------------------------------------------------
# verify attention sweep (9B-like, 2048 cached)
# ---------------------------------------------------------------------------

def verify_sweep(layers=ROT_LAYERS, reps=3):
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
        best = math.inf
        for _ in range(reps):
            st.kv_truncate(0, P)
            with Timer() as t:
                for layer in range(layers):
                    st.extend_attn(0, layer, qm, km, vm, out)
            best = min(best, t.ms / layers)
        res[m] = dict(us=best * 1e3,
                      GBps=attn_bytes(P, m, hq, hkv, d) / (best * 1e-3) / 1e9)
    return res


# ---------------------------------------------------------------------------
# MoE routed GEMV (35B-A3B-like)
# ---------------------------------------------------------------------------

def moe_sweep(reps=3, n_routings=16, sets=2):
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

        def run():
            for i in range(n_routings):
                s = i % sets
                sve.w4_gemv_m_routed(x, ids[i], W1[s], E, n1, k1, False, y1)
                sve.w4_gemv_m_routed(h, ids[i], W2[s], E, n2, k2, True, y2)
        run()
        best = math.inf
        for _ in range(reps):
            with Timer() as t:
                run()
            best = min(best, t.ms / n_routings)
        ub = float(np.mean(union)) * (eb1 + eb2)
        res[m] = dict(us=best * 1e3, union_experts=float(np.mean(union)),
                      GBps=ub / (best * 1e-3) / 1e9)
    return res


# ---------------------------------------------------------------------------
# four slots in rotation (4B-like), batched extend
# ---------------------------------------------------------------------------

def slots_rotation():
    wl = synth.WORKLOADS["slots4b"]
    hq, hkv, d = wl["hq"], wl["hkv"], wl["d"]
    st = sve.KVSlots(4, 1, hq, hkv, d, 1024, 4 * 1024)
    order = synth.rotation_sessions(wl["seed"], 4, wl["turns"], wl["state_tokens"],
                                    wl["shared_start"], wl["question_min"], wl["question_max"])
    g = synth.rng(wl["seed"], 88)
    prefilled, times, toks = [], [], 0
    # first round: fill the four 800+ token states
    for rnd in range(wl["turns"]):
        reqs = order[4 * rnd:4 * rnd + 4]
        sel = [st.kv_slot_select(p) for _, p in reqs]
        ms = [len(p) - r for (_, p), (_, r) in zip(reqs, sel)]
        prefilled.append(ms)
        total = sum(ms)
        q, k, v = (bf16_dev(a) for a in synth.attention_rows(g, total, hq, hkv, d))
        with Timer() as t:
            st.extend_attn_batched([s for s, _ in sel], ms, 0, q, k, v)
        if rnd > 0:
            times.append(t.ms)
            toks += total
    return dict(prefilled_per_turn=prefilled,
                batched_tok_per_s=toks / (sum(times) * 1e-3) if times else None,
                ms_per_round=float(np.median(times)) if times else None)


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(case, P, budget_s=10.0):
    from oracle.attention import extend_attention
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
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
                       f"new rows, fp64 numpy), repeated {n}x over {budget_s:.0f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the GEMV / verify / MoE / slot sweeps")
    ap.add_argument("--layers", type=int, default=ROT_LAYERS)
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the copy probe (256 MiB, three times): the known byte count "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.calibrate:
        torch.cuda.set_device(0)
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            sve.probe_copy(src, dst, 4096)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": src.numel(), "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is not sharded); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    sve.load_library()

    print("[bench] replay setup", file=sys.stderr, flush=True)
    rp = Replay(args.layers)
    # eager: every layer's extend launched from Python
    for _ in range(args.warmup):
        rp.step()
    torch.cuda.synchronize()
    with Timer() as t:
        for _ in range(args.steps):
            rp.step()
    ms_eager = t.ms / args.steps
    # graph: the same calls captured once and replayed
    rp.capture()
    for _ in range(args.warmup):
        rp.step_graph()
    torch.cuda.synchronize()
    with Timer() as t:
        for _ in range(args.steps):
            rp.step_graph()
    ms_step = t.ms / args.steps
    per_layer_s = ms_step * 1e-3 / args.layers
    value = rp.m / per_layer_s
    print(f"[bench] step {ms_step:.3f} ms (eager {ms_eager:.3f}), {per_layer_s * 1e6:.2f} us per "
          "layer", file=sys.stderr, flush=True)

    ext_ms = rp.time_extend_graph()
    flops = attn_flops(rp.P, rp.m, rp.hq, rp.d)
    achieved = flops / (ext_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None,
                "kernel": "one extend call (kv_append + attn_mfma + combine kernels), 1668+254, "
                          "28/4 heads, D 128, timed by HIP events over graph replays",
                "us_per_launch": round(ext_ms * 1e3, 2), "flops_per_launch": flops}

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tok/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "agent-turn replay turn 9: select + extend of 254 new rows over "
                                  "1668 cached, 7B-like attention layer (28 q / 4 KV heads, D 128), "
                                  f"{args.layers} layers rotated, per-layer calls replayed from a "
                                  "captured HIP graph; value = tokens per layer pass",
                      "global_batch": rp.m, "seq_len": rp.n, "parallelism": "none",
                      "ms_per_step_eager": round(ms_eager, 4)},
           "roofline": roofline}

    if not args.no_extra:
        print("[bench] gemv sweep", file=sys.stderr, flush=True)
        g9 = gemv_sweep(synth.layer_gemv_shapes(4096, 12288, 32, 8, 128))
        g7 = gemv_sweep(synth.layer_gemv_shapes(3584, 18944, 28, 4, 128), copies=6, m_values=(1, 4, 8))
        a, b = fit(list(g9), [g9[m]["us"] for m in g9])
        worst = min(v["GBps"] for v in g9.values())
        out["gemv"] = {
            "workload": "9B-like layer (QKV 6144x4096, O 4096x4096, gate|up 24576x4096, "
                        "down 4096x12288), int4 group-32, 8 rotated copies",
            "GBps_min_over_m": round(worst, 1), "frac_of_hbm_peak_min": round(worst / HBM_PEAK_GBS, 4),
            "per_m": {m: {"us": round(v["us"], 2), "GBps": round(v["GBps"], 1),
                          "frac": round(v["GBps"] / HBM_PEAK_GBS, 4)} for m, v in g9.items()},
            "fit_us": {"fixed": round(a, 3), "per_row": round(b, 3), "per_row_over_fixed": round(b / a, 4)},
            "7b_layer_per_m": {m: {"us": round(v["us"], 2), "GBps": round(v["GBps"], 1)} for m, v in g7.items()},
        }
        print("[bench] verify sweep", file=sys.stderr, flush=True)
        vs = verify_sweep(layers=min(args.layers, ROT_LAYERS))
        a2, b2 = fit(list(vs), [vs[m]["us"] for m in vs])
        out["verify_attention"] = {
            "workload": "9B-like attention (32 q / 8 KV heads, D 128), 2048 cached + m rows",
            "per_m": {m: {"us": round(v["us"], 2), "GBps": round(v["GBps"], 1)} for m, v in vs.items()},
            "fit_us": {"fixed": round(a2, 3), "per_row": round(b2, 3)}}
        # the same sweep with each kernel path forced, as evidence for the
        # default path choice
        for path, rows in (("valu", "100000"), ("mfma", "1")):
            os.environ["SVE_MFMA_MIN_ROWS"] = rows
            vp = verify_sweep(layers=32, reps=2)
            out["verify_attention"]["forced_" + path] = {m: round(v["us"], 2) for m, v in vp.items()}
        os.environ.pop("SVE_MFMA_MIN_ROWS", None)
        print("[bench] moe sweep", file=sys.stderr, flush=True)
        mo = moe_sweep()
        a3, b3 = fit(list(mo), [mo[m]["us"] for m in mo])
        out["moe"] = {
            "workload": "35B-A3B-like expert layer: 256 experts, W1 1024x2048, W2 2048x512, top-8",
            "per_m": {m: {"us": round(v["us"], 2), "union_experts": round(v["union_experts"], 2),
                          "GBps": round(v["GBps"], 1)} for m, v in mo.items()},
            "fit_us": {"fixed": round(a3, 3), "per_row": round(b3, 3)}}
        print("[bench] slots", file=sys.stderr, flush=True)
        out["slots"] = slots_rotation()

    if not args.no_cpu:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(rp.case, rp.P)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
