"""Extend calls captured in a HIP graph and replayed, as the bench times
them: every replay gives bitwise the outputs of the eager calls, with eager
work and synchronizations between the replays. A replay repeats the kernels
only (the host's row counts advance when the calls are made, at capture),
so the rows a replay appends are checked through a second extend in the
same graph that reads them as cached keys. The eager outputs and appended
rows are checked against the oracle and the inputs."""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle.attention import extend_attention
from tests.gpu_helpers import announce, dev_bf16, host_bits, require_gpu

pytestmark = pytest.mark.gpu
ATTN_TOL = 1e-2


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def test_graph_replays_match_eager_calls():
    hq, hkv, d, P, m, layers = 28, 4, 128, 1668, 254, 2
    m2 = 8  # rows of a follow-up extend that reads the appended rows
    mv, Pv = 4, 900  # a verify-sized call on a second slot (decode kernel + combine)
    announce(f"graph replay turn9 layers={layers} + verify m={mv}")
    st = sve.KVSlots(2, layers, hq, hkv, d, 2112, P)
    c = synth.attention_case(2, hq, hkv, d, P, m)
    cv = synth.attention_case(5, hq, hkv, d, Pv, mv)
    toks = np.arange(P + m + m2, dtype=np.int32)
    q2, k2, v2 = synth.attention_rows(synth.rng(6), m2, hq, hkv, d)
    toks_v = np.arange(10_000, 10_000 + Pv + mv, dtype=np.int32)
    assert st.kv_slot_select(toks[:P]) == (0, 0)
    for layer in range(layers):
        st.extend_attn(0, layer, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                       dev_bf16(c["v_prefix"]))
    assert st.kv_slot_select(toks_v[:Pv]) == (1, 0)
    for layer in range(layers):
        st.extend_attn(1, layer, dev_bf16(cv["q_prefix"]), dev_bf16(cv["k_prefix"]),
                       dev_bf16(cv["v_prefix"]))
    q, k, v = dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"])
    qv, kv, vv = dev_bf16(cv["q"]), dev_bf16(cv["k"]), dev_bf16(cv["v"])
    q2d, k2d, v2d = dev_bf16(q2), dev_bf16(k2), dev_bf16(v2)
    outs = [torch.empty_like(q) for _ in range(layers)]
    outs2 = [torch.empty_like(q2d) for _ in range(layers)]
    out_v = torch.empty_like(qv)

    def select():
        st.kv_truncate(0, P)
        st.kv_truncate(1, Pv)
        assert st.kv_slot_select(toks) == (0, P)
        assert st.kv_slot_select(toks_v) == (1, Pv)

    def calls():
        for layer in range(layers):
            st.extend_attn(0, layer, q, k, v, outs[layer])
            st.extend_attn(0, layer, q2d, k2d, v2d, outs2[layer])
        st.extend_attn(1, layers - 1, qv, kv, vv, out_v)

    def snapshot():
        torch.cuda.synchronize()
        return ([host_bits(o) for o in outs], [host_bits(o) for o in outs2], host_bits(out_v))

    select()
    calls()
    ref_out, ref_out2, ref_v = snapshot()
    f64 = lambda bits: synth.bf16_bits_to_f32(bits).astype(np.float64)
    k_all = np.concatenate([c["k_prefix"], c["k"], k2])
    v_all = np.concatenate([c["v_prefix"], c["v"], v2])
    want = extend_attention(c["q"], k_all[:P + m], v_all[:P + m], P)
    want2 = extend_attention(q2, k_all, v_all, P + m)
    for layer in range(layers):
        assert np.abs(f64(ref_out[layer]) - want).max() <= ATTN_TOL
        assert np.abs(f64(ref_out2[layer]) - want2).max() <= ATTN_TOL
        kk, vv_ = st.kv_read(0, layer, P, m + m2)
        assert np.array_equal(host_bits(kk), k_all[P:])
        assert np.array_equal(host_bits(vv_), v_all[P:])
    want_v = extend_attention(cv["q"], np.concatenate([cv["k_prefix"], cv["k"]]),
                              np.concatenate([cv["v_prefix"], cv["v"]]), Pv)
    assert np.abs(f64(ref_v) - want_v).max() <= ATTN_TOL

    select()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        calls()
    torch.cuda.synchronize()

    g = synth.rng(7)
    for rep in range(3):
        announce(f"graph replay {rep}")
        # eager work between replays: clear the outputs, run an extend of
        # other rows on the second slot, synchronize
        for o in outs + outs2:
            o.zero_()
        out_v.zero_()
        st.kv_truncate(1, Pv)
        assert st.kv_slot_select(toks_v) == (1, Pv)
        junk = [dev_bf16(a) for a in synth.attention_rows(g, mv, hq, hkv, d)]
        st.extend_attn(1, 0, *junk)
        torch.cuda.synchronize()
        select()
        graph.replay()
        got_out, got_out2, got_v = snapshot()
        for layer in range(layers):
            assert np.array_equal(got_out[layer], ref_out[layer]), (rep, layer)
            assert np.array_equal(got_out2[layer], ref_out2[layer]), (rep, layer)
        assert np.array_equal(got_v, ref_v), rep
