"""GPU regression tests for three fixed defects of the extend path, each run
against the fp64 oracle through the C ABI:

- a cut-back slot keeps stale rows past its cached length (goinfer, "Turn nine
  in under half a second", "How it works": the conversation is cut back to the
  shared point and only the rest is prefilled). No kernel may let those rows
  reach an output: a masked key has probability 0, but 0 times a stale
  non-finite value is NaN.
- several questions about one state append nothing (openjev-multimodal,
  "Latency", "What changed": prefix priming keeps the state), also with one
  question and when the questions run past the slot's capacity.
- a batched call of decode-sized pieces with few KV heads plans its key
  splits within the split workspace (the slot rows after it stay intact).

And one guard for the split partials, which leave the attention kernel by
stores that write through the L2: consecutive split calls on one context,
each over the same workspace, read only their own partials.
"""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle.attention import extend_attention, extend_attention_questions
from tests.gpu_helpers import announce, dev_bf16, env, host_bits, host_f64_of_bf16, require_gpu

pytestmark = pytest.mark.gpu
ATTN_TOL = 1e-2  # max-abs against the fp64 oracle

BF16_NAN, BF16_INF, BF16_NINF = 0x7FC0, 0x7F80, 0xFF80


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _slot_region(st: sve.KVSlots, n_layers: int = 1) -> np.ndarray:
    """Bytes of every slot's K/V store: the arena ends with the slots, each
    n_layers x {K [Hkv][cap][D], Vt [Hkv][D][cap]} bf16 (256-byte aligned)."""
    layer = (2 * st.hkv * st.capacity * st.d * 2 + 255) // 256 * 256
    n = st.requested * n_layers * layer
    return st.arena[-n:].cpu().numpy().copy()


def _junk(shape, seed):
    """bf16 rows of NaN, +Inf and -Inf."""
    r = np.random.default_rng(seed)
    return r.choice(np.array([BF16_NAN, BF16_INF, BF16_NINF], dtype=np.uint16), size=shape)


STALE_PATHS = {
    "decode": dict(SVE_ATTN_PATH="decode"),
    "decode-split5": dict(SVE_ATTN_PATH="decode", SVE_KV_SPLIT=5),
    "mfma": dict(SVE_MFMA_MIN_ROWS=1),
    "mfma-split3": dict(SVE_MFMA_MIN_ROWS=1, SVE_KV_SPLIT=3),
    "mfma-separate-append": dict(SVE_MFMA_MIN_ROWS=1, SVE_FUSED_APPEND=0),
    "valu": dict(SVE_MFMA_MIN_ROWS=100000),
    "rows": dict(SVE_ATTN_PATH="rows"),
    "rows-separate-append": dict(SVE_ATTN_PATH="rows", SVE_FUSED_APPEND=0),
}


@pytest.mark.parametrize("path", list(STALE_PATHS))
@pytest.mark.parametrize("case", [(32, 8, 128, 333, 3), (32, 8, 128, 2061, 8), (4, 2, 64, 45, 5),
                                  (28, 4, 128, 1000, 40)],
                         ids=lambda c: "h%d-%d-d%d-P%d-m%d" % c)
def test_stale_nonfinite_rows_past_the_cut_never_reach_outputs(case, path):
    """Fill a slot, extend 64 rows whose K and V are NaN or infinite, cut back
    to P (P % 32 != 0), then extend m rows: outputs finite and within the
    tolerance of the oracle, which never sees the junk rows."""
    hq, hkv, d, P, m = case
    if path.startswith("decode") and m * (hq // hkv) > 64:
        pytest.skip("decode path takes at most 64 packed rows")
    announce(f"stale rows past P {case} path={path}")
    assert P % 32 != 0
    c = synth.attention_case(200 + P, hq, hkv, d, P, m)
    st = sve.KVSlots(1, 1, hq, hkv, d, P + 64 + 64, max(P, 64))
    assert st.kv_slot_select(np.arange(P + 64, dtype=np.int32)) == (0, 0)
    st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]), dev_bf16(c["v_prefix"]))
    jq = synth.normal_bf16(synth.rng(7, P), (64, hq, d))
    st.extend_attn(0, 0, dev_bf16(jq), dev_bf16(_junk((64, hkv, d), 1)),
                   dev_bf16(_junk((64, hkv, d), 2)))
    st.kv_truncate(0, P)
    with env(**STALE_PATHS[path]):
        out = st.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]))
    got = host_f64_of_bf16(out)
    want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                            np.concatenate([c["v_prefix"], c["v"]]), P)
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= ATTN_TOL
    # the new rows replaced the junk at P .. P+m-1
    k_new, v_new = st.kv_read(0, 0, P, m)
    assert np.array_equal(host_bits(k_new), c["k"]) and np.array_equal(host_bits(v_new), c["v"])


@pytest.mark.parametrize("fused", [1, 0], ids=["fused", "separate-append"])
@pytest.mark.parametrize("ms", [[56], [100], [30, 70]], ids=["one-fills-cap", "one-past-cap",
                                                           "two-past-cap"])
def test_questions_never_append_even_past_capacity(ms, fused):
    """A slot of capacity 256 holding 200 rows; questions of 56 rows (ending
    exactly at the capacity), 100 rows, or 30 + 70 rows (running past it).
    Every byte of the slot store is unchanged, the cached length stays 200,
    and the outputs match the oracle."""
    hq, hkv, d, P = 8, 2, 128, 200
    total = int(sum(ms))
    announce(f"questions {ms} past capacity fused={fused}")
    c = synth.attention_case(300 + total, hq, hkv, d, P, total)
    st = sve.KVSlots(1, 1, hq, hkv, d, 256, 256)
    assert st.capacity == 256
    assert st.kv_slot_select(np.arange(P, dtype=np.int32)) == (0, 0)
    st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]), dev_bf16(c["v_prefix"]))
    torch.cuda.synchronize()
    before = _slot_region(st)
    with env(SVE_FUSED_APPEND=fused):
        out = st.extend_attn_questions(0, 0, ms, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                       dev_bf16(c["v"]))
    torch.cuda.synchronize()
    after = _slot_region(st)
    want = extend_attention_questions(c["q"], c["k_prefix"], c["v_prefix"], c["k"], c["v"], ms)
    assert np.abs(host_f64_of_bf16(out) - want).max() <= ATTN_TOL
    assert st.kv_len(0, 0) == P
    assert np.array_equal(before, after)


def test_batched_decode_pieces_fit_the_split_workspace():
    """Four decode-sized pieces (8 rows, 2 KV heads of 2 query heads each)
    over 3000 cached rows, with max_rows = 32 = the call's rows: every piece
    has a cached split and its new-key split, and the plan stays within the
    16 x 32 rows of split workspace. Outputs match the oracle and every
    cached row of every slot is still the one appended."""
    hq, hkv, d, P, m = 4, 2, 64, 3000, 8
    announce("batched decode pieces, few KV heads, P=3000")
    st = sve.KVSlots(4, 1, hq, hkv, d, P + m, 4 * m)
    cases = [synth.attention_case(400 + s, hq, hkv, d, P, m) for s in range(4)]
    for s in range(4):
        toks = np.arange(P + m, dtype=np.int32) + 10000 * (s + 1)
        assert st.kv_slot_select(toks) == (s, 0)
    chunk = 32
    for s, c in enumerate(cases):  # prefill in calls of at most max_rows rows
        for r in range(0, P, chunk):
            e = min(P, r + chunk)
            st.extend_attn(s, 0, dev_bf16(c["q_prefix"][r:e]), dev_bf16(c["k_prefix"][r:e]),
                           dev_bf16(c["v_prefix"][r:e]))
    q = np.concatenate([c["q"] for c in cases])
    k = np.concatenate([c["k"] for c in cases])
    v = np.concatenate([c["v"] for c in cases])
    with env(SVE_LOG=0):
        out = host_f64_of_bf16(st.extend_attn_batched([0, 1, 2, 3], [m] * 4, 0, dev_bf16(q),
                                                      dev_bf16(k), dev_bf16(v)))
    for s, c in enumerate(cases):
        want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                                np.concatenate([c["v_prefix"], c["v"]]), P)
        assert np.abs(out[s * m:(s + 1) * m] - want).max() <= ATTN_TOL
        kk, vv = st.kv_read(s, 0, 0, P + m)
        assert np.array_equal(host_bits(kk), np.concatenate([c["k_prefix"], c["k"]]))
        assert np.array_equal(host_bits(vv), np.concatenate([c["v_prefix"], c["v"]]))


@pytest.mark.parametrize("path", ["mfma-split5", "mfma-balanced", "decode-split3"])
def test_consecutive_split_calls_read_only_their_own_partials(path):
    """One slot holding 1668 rows; six extends in a row, each cut back to
    the same 1668 rows first, with fresh q/k/v of alternating sizes (254,
    37, 254, 8, 254, 3 rows on the MFMA path; 8, 3, 8, 1, 8, 5 on the decode
    path), every one on a split layout over the same workspace. Each output
    matches the oracle of its own inputs: no call's combine reads a partial
    of an earlier call."""
    hq, hkv, d, P = 28, 4, 128, 1668
    env_of = {"mfma-split5": dict(SVE_MFMA_MIN_ROWS=1, SVE_KV_SPLIT=5),
              "mfma-balanced": dict(SVE_MFMA_MIN_ROWS=1, SVE_ATTN_LAYOUT=3),
              "decode-split3": dict(SVE_ATTN_PATH="decode", SVE_KV_SPLIT=3)}[path]
    ms = [8, 3, 8, 1, 8, 5] if path.startswith("decode") else [254, 37, 254, 8, 254, 3]
    announce(f"consecutive split calls path={path}")
    base = synth.attention_case(500, hq, hkv, d, P, 0)
    st = sve.KVSlots(1, 1, hq, hkv, d, P + 256 + 64, P)
    assert st.kv_slot_select(np.arange(P + 256, dtype=np.int32)) == (0, 0)
    st.extend_attn(0, 0, dev_bf16(base["q_prefix"]), dev_bf16(base["k_prefix"]),
                   dev_bf16(base["v_prefix"]))
    for i, m in enumerate(ms):
        st.kv_truncate(0, P)
        c = synth.attention_case(600 + i, hq, hkv, d, 0, m)
        with env(**env_of):
            out = st.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]))
        got = host_f64_of_bf16(out)
        want = extend_attention(c["q"], np.concatenate([base["k_prefix"], c["k"]]),
                                np.concatenate([base["v_prefix"], c["v"]]), P)
        assert np.abs(got - want).max() <= ATTN_TOL, (i, m)
