"""GPU parity of extend-prefill attention against the oracle (max-abs 1e-2,
bf16 in/out, fp32 accumulation), on both kernel paths, with and without key
splits, plus the invariants the pages fix: extend over a cached prefix equals
the tail of a full prefill, token-by-token equals one pass, and the cached
K/V rows are exactly the appended ones."""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle.attention import extend_attention
from tests.gpu_helpers import (announce, dev_bf16, env, host_bits, host_f64_of_bf16,
                               require_gpu)

pytestmark = pytest.mark.gpu
ATTN_TOL = 1e-2  # max-abs against the fp64 oracle

PATHS = {"valu": dict(SVE_MFMA_MIN_ROWS=100000), "mfma": dict(SVE_MFMA_MIN_ROWS=1),
         "decode": dict(SVE_ATTN_PATH="decode"),  # decode: pieces of <= 64 packed rows
         "rows": dict(SVE_ATTN_PATH="rows")}      # row tiles over every key, no split
ALL_PATHS = ["valu", "mfma", "decode", "rows"]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _store(hq, hkv, d, cap, max_rows, n_slots=1, n_layers=1):
    return sve.KVSlots(n_slots, n_layers, hq, hkv, d, cap, max_rows)


def _run_case(hq, hkv, d, prefix, m, path, seed=0, split=0, prefill_path=None):
    """Fill a slot with `prefix` rows, then extend by m rows; returns
    (gpu output of the m rows, oracle output, case dict)."""
    c = synth.attention_case(seed, hq, hkv, d, prefix, m)
    st = _store(hq, hkv, d, prefix + m + 64, max(prefix, m, 1))
    toks = np.arange(prefix + m, dtype=np.int32)
    slot, reused = st.kv_slot_select(toks)
    assert (slot, reused) == (0, 0)
    # (path None: the library's own choice)
    if prefix:
        with env(**PATHS.get(prefill_path or path, {})):
            st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                           dev_bf16(c["v_prefix"]))
    with env(SVE_KV_SPLIT=split, **PATHS.get(path, {})):
        out = st.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]))
    k_all = np.concatenate([c["k_prefix"], c["k"]])
    v_all = np.concatenate([c["v_prefix"], c["v"]])
    want = extend_attention(c["q"], k_all, v_all, prefix)
    return host_f64_of_bf16(out), want, c, st


CASES = [
    # hq, hkv, d, prefix, m
    (4, 2, 64, 64, 8),      # tiny single layer: 64 cached + 8 new rows
    (4, 2, 64, 0, 64),      # tiny prefix fill (full prefill)
    (4, 2, 64, 0, 1),       # one row, one key
    (8, 8, 128, 100, 13),   # no GQA, ragged prefix
    (28, 4, 128, 200, 37),  # 7B-like heads, ragged rows
    (32, 8, 128, 130, 5),   # 9B-like heads, verify-sized suffix
    (4, 1, 128, 300, 70),   # wide group, several row blocks
]


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "h%d-%d-d%d-P%d-m%d" % c)
def test_extend_matches_oracle(case, path):
    hq, hkv, d, prefix, m = case
    announce(f"extend {case} path={path}")
    got, want, _, _ = _run_case(hq, hkv, d, prefix, m, path)
    assert np.abs(got - want).max() <= ATTN_TOL


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("split", [1, 2, 5, 16])
def test_key_splits(path, split):
    announce(f"splits={split} path={path}")
    got, want, _, _ = _run_case(8, 2, 128, 700, 21, path, seed=3, split=split)
    assert np.abs(got - want).max() <= ATTN_TOL


@pytest.mark.parametrize("split", [1, 3, 12, 40, 64])
@pytest.mark.parametrize("m", [1, 6])
def test_decode_key_splits(m, split):
    """Decode path (verify-sized pieces) with forced key splits, up to the
    path's 64-split limit, including splits that hold only cached rows."""
    announce(f"decode splits={split} m={m}")
    got, want, _, _ = _run_case(32, 8, 128, 1500, m, "decode", seed=12, split=split)
    assert np.abs(got - want).max() <= ATTN_TOL


def test_decode_batched_matches_single_slot_calls():
    """Four verify-sized pieces (m = 1, 3, 8, 5 on 9B-like heads) in one
    decode launch equal four separate calls and the oracle."""
    hq, hkv, d = 32, 8, 128
    Ps, ms = [700, 1030, 64, 1900], [1, 3, 8, 5]
    sts = [sve.KVSlots(4, 1, hq, hkv, d, 2048, 2048) for _ in range(2)]
    cases = [synth.attention_case(50 + i, hq, hkv, d, Ps[i], ms[i]) for i in range(4)]
    announce("decode batched")
    for st in sts:
        for i in range(4):
            toks = np.concatenate([[i + 1], np.arange(Ps[i] + ms[i] - 1)]).astype(np.int32)
            slot, r = st.kv_slot_select(toks)
            assert (slot, r) == (i, 0)
            st.extend_attn(slot, 0, dev_bf16(cases[i]["q_prefix"]),
                           dev_bf16(cases[i]["k_prefix"]), dev_bf16(cases[i]["v_prefix"]))
    q = dev_bf16(np.concatenate([c["q"] for c in cases]))
    k = dev_bf16(np.concatenate([c["k"] for c in cases]))
    v = dev_bf16(np.concatenate([c["v"] for c in cases]))
    with env(**PATHS["decode"]):
        out_b = host_f64_of_bf16(sts[0].extend_attn_batched([0, 1, 2, 3], ms, 0, q, k, v))
    row = 0
    for i in range(4):
        c = cases[i]
        with env(**PATHS["decode"]):
            single = host_f64_of_bf16(sts[1].extend_attn(i, 0, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                                         dev_bf16(c["v"])))
        want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                                np.concatenate([c["v_prefix"], c["v"]]), Ps[i])
        part = out_b[row:row + ms[i]]
        assert np.abs(part - want).max() <= ATTN_TOL
        assert np.abs(part - single).max() <= ATTN_TOL
        row += ms[i]
    for st in sts:
        for i in range(4):
            kk, vv = st.kv_read(i, 0, Ps[i], ms[i])
            assert np.array_equal(host_bits(kk), cases[i]["k"])
            assert np.array_equal(host_bits(vv), cases[i]["v"])


def test_turn9_full_size():
    """Agent-turn replay turn 9: 1668 cached + 254 new rows, 28 q / 4 KV heads,
    D 128, default launch configuration (the one the bench times)."""
    announce("turn9 full")
    got, want, _, _ = _run_case(28, 4, 128, 1668, 254, None, seed=2)
    assert np.abs(got - want).max() <= ATTN_TOL


@pytest.mark.parametrize("path", ["mfma", "rows"])
def test_turn9_full_size_each_path(path):
    """Turn 9 on each of the two many-row kernels, forced."""
    announce(f"turn9 full path={path}")
    got, want, _, _ = _run_case(28, 4, 128, 1668, 254, path, seed=2)
    assert np.abs(got - want).max() <= ATTN_TOL


@pytest.mark.parametrize("case", [(28, 4, 128, 1664, 254), (28, 4, 128, 1668, 254),
                                  (8, 2, 128, 63, 300), (4, 1, 64, 130, 129),
                                  (8, 2, 128, 0, 200), (8, 2, 128, 700, 21)],
                         ids=lambda c: "h%d-%d-d%d-P%d-m%d" % c)
@pytest.mark.parametrize("path", ["mfma", "rows"])
def test_in_kernel_append_matches_separate_append(case, path):
    """MFMA and row-tile paths: the attention kernel reads the new rows from
    the call's inputs and appends them itself (the default), or a separate
    append kernel writes them first. Both match the oracle, and the cached
    rows they leave are the appended rows, bit for bit."""
    hq, hkv, d, P, m = case
    for fused in (1, 0):
        announce(f"in-kernel append={fused} {case} path={path}")
        with env(SVE_FUSED_APPEND=fused):
            got, want, c, st = _run_case(hq, hkv, d, P, m, path, seed=13)
        assert np.abs(got - want).max() <= ATTN_TOL
        kk, vv = st.kv_read(0, 0, 0, P + m)
        assert np.array_equal(host_bits(kk), np.concatenate([c["k_prefix"], c["k"]]))
        assert np.array_equal(host_bits(vv), np.concatenate([c["v_prefix"], c["v"]]))


@pytest.mark.parametrize("m", list(range(1, 9)))
def test_verify_full_size(m):
    """Speculative verify: 2048 cached + m rows, 32 q / 8 KV heads, D 128, on
    the default path for that m."""
    announce(f"verify full m={m}")
    c = synth.attention_case(3, 32, 8, 128, 2048, m)
    st = _store(32, 8, 128, 2048 + 8, 2048)
    st.kv_slot_select(np.arange(2048 + m, dtype=np.int32))
    st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]), dev_bf16(c["v_prefix"]))
    out = st.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]))
    want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                            np.concatenate([c["v_prefix"], c["v"]]), 2048)
    assert np.abs(host_f64_of_bf16(out) - want).max() <= ATTN_TOL


@pytest.mark.parametrize("path", ALL_PATHS)
def test_extend_equals_tail_of_full_prefill(path):
    """Extend over a cached prefix == the last rows of a from-scratch prefill
    of the whole sequence, both on the GPU."""
    hq, hkv, d, P, m = 8, 2, 128, 150, 30
    announce(f"tail-of-prefill path={path}")
    got, _, c, _ = _run_case(hq, hkv, d, P, m, path, seed=5)
    st = _store(hq, hkv, d, P + m + 64, P + m)
    st.kv_slot_select(np.arange(P + m, dtype=np.int32))
    with env(**PATHS[path]):
        full = st.extend_attn(0, 0, dev_bf16(np.concatenate([c["q_prefix"], c["q"]])),
                              dev_bf16(np.concatenate([c["k_prefix"], c["k"]])),
                              dev_bf16(np.concatenate([c["v_prefix"], c["v"]])))
    assert np.abs(host_f64_of_bf16(full)[P:] - got).max() <= ATTN_TOL


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_token_by_token_equals_one_pass_bitwise(path):
    """Within one kernel path and without key splits, m one-row calls give the
    same bits as one m-row call: each row's arithmetic depends only on its own
    query and the keys it sees, in absolute-position tile order. (The decode
    path splits at the cached length, which moves with each call; it is
    checked to tolerance below.)"""
    hq, hkv, d, P, m = 8, 2, 128, 90, 12
    c = synth.attention_case(7, hq, hkv, d, P, m)
    announce(f"token-by-token path={path}")
    outs = []
    for mode in ("one", "many"):
        st = _store(hq, hkv, d, P + m + 64, P + m)
        st.kv_slot_select(np.arange(P + m, dtype=np.int32))
        with env(SVE_KV_SPLIT=1, **PATHS[path]):
            st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                           dev_bf16(c["v_prefix"]))
            if mode == "one":
                outs.append(host_bits(st.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                                     dev_bf16(c["v"]))))
            else:
                rows = [host_bits(st.extend_attn(0, 0, dev_bf16(c["q"][i:i + 1]),
                                                 dev_bf16(c["k"][i:i + 1]),
                                                 dev_bf16(c["v"][i:i + 1]))) for i in range(m)]
                outs.append(np.concatenate(rows))
    assert np.array_equal(outs[0], outs[1])


def test_decode_token_by_token_matches_one_pass():
    """Decode path: m one-row calls (each splitting at its own cached length)
    agree with one m-row call and with the oracle within tolerance."""
    hq, hkv, d, P, m = 32, 8, 128, 300, 8
    c = synth.attention_case(13, hq, hkv, d, P, m)
    announce("decode token-by-token")
    outs = []
    for mode in ("one", "many"):
        st = _store(hq, hkv, d, P + m + 64, P + m)
        st.kv_slot_select(np.arange(P + m, dtype=np.int32))
        st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                       dev_bf16(c["v_prefix"]))
        with env(**PATHS["decode"]):
            if mode == "one":
                outs.append(host_f64_of_bf16(st.extend_attn(0, 0, dev_bf16(c["q"]),
                                                            dev_bf16(c["k"]), dev_bf16(c["v"]))))
            else:
                outs.append(np.concatenate([
                    host_f64_of_bf16(st.extend_attn(0, 0, dev_bf16(c["q"][i:i + 1]),
                                                    dev_bf16(c["k"][i:i + 1]),
                                                    dev_bf16(c["v"][i:i + 1])))
                    for i in range(m)]))
    want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                            np.concatenate([c["v_prefix"], c["v"]]), P)
    assert np.abs(outs[0] - outs[1]).max() <= 2 * ATTN_TOL
    for o in outs:
        assert np.abs(o - want).max() <= ATTN_TOL


def test_paths_agree_within_tolerance():
    """The VALU and MFMA paths differ only by rounding (bf16 probabilities in
    the MFMA value product); both stay within the oracle tolerance."""
    announce("paths agree")
    a, want, _, _ = _run_case(16, 4, 128, 400, 9, "valu", seed=8)
    b, _, _, _ = _run_case(16, 4, 128, 400, 9, "mfma", seed=8)
    c, _, _, _ = _run_case(16, 4, 128, 400, 9, "decode", seed=8)
    for x in (b, c):
        assert np.abs(a - x).max() <= 2 * ATTN_TOL
    for x in (a, b, c):
        assert np.abs(x - want).max() <= ATTN_TOL


@pytest.mark.parametrize("path", ALL_PATHS)
def test_cached_rows_are_the_appended_rows(path):
    hq, hkv, d, P, m = 4, 2, 64, 70, 9
    announce(f"kv read path={path}")
    _, _, c, st = _run_case(hq, hkv, d, P, m, path, seed=9)
    k, v = st.kv_read(0, 0, 0, P + m)
    assert np.array_equal(host_bits(k), np.concatenate([c["k_prefix"], c["k"]]))
    assert np.array_equal(host_bits(v), np.concatenate([c["v_prefix"], c["v"]]))


@pytest.mark.parametrize("path", ["mfma", "rows"])
def test_deterministic_repeats(path):
    hq, hkv, d, P, m = 28, 4, 128, 500, 60
    c = synth.attention_case(10, hq, hkv, d, P, m)
    st = _store(hq, hkv, d, P + m + 64, P + m)
    st.kv_slot_select(np.arange(P + m, dtype=np.int32))
    st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]), dev_bf16(c["v_prefix"]))
    q, k, v = dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"])
    announce(f"determinism path={path}")
    with env(**PATHS[path]):
        first = st.extend_attn(0, 0, q, k, v)
        for _ in range(100):
            st.kv_truncate(0, P)
            assert torch.equal(st.extend_attn(0, 0, q, k, v), first)


def test_zero_rows_is_noop_and_state_errors():
    st = _store(4, 2, 64, 128, 64)
    z = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    st.kv_slot_select(np.arange(10, dtype=np.int32))
    st.extend_attn(0, 0, z, zk, zk)
    assert st.kv_len(0) == 0
    q = torch.zeros((11, 4, 64), dtype=torch.bfloat16, device="cuda")
    kk = torch.zeros((11, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sve.SveError) as e:
        st.extend_attn(0, 0, q, kk, kk)  # 11 rows > the 10 selected tokens
    assert e.value.code == -5
    with pytest.raises(sve.SveError) as e:
        st.extend_attn(1, 0, q[:1], kk[:1], kk[:1])
    assert e.value.code == -2


def test_batched_matches_single_slot_calls():
    """Four slots in one launch (4B-like heads, ~30-row questions on
    ~800-token states) equal four separate calls and the oracle."""
    hq, hkv, d = 32, 8, 128
    Ps, ms = [800, 830, 861, 905], [30, 24, 36, 27]
    st_b = sve.KVSlots(4, 1, hq, hkv, d, 1024, 1024)
    st_s = sve.KVSlots(4, 1, hq, hkv, d, 1024, 1024)
    cases = [synth.attention_case(40 + i, hq, hkv, d, Ps[i], ms[i]) for i in range(4)]
    announce("batched")
    for st in (st_b, st_s):
        for i in range(4):
            toks = np.concatenate([[i + 1], np.arange(Ps[i] + ms[i] - 1)]).astype(np.int32)
            slot, r = st.kv_slot_select(toks)
            assert (slot, r) == (i, 0)
            st.extend_attn(slot, 0, dev_bf16(cases[i]["q_prefix"]),
                           dev_bf16(cases[i]["k_prefix"]), dev_bf16(cases[i]["v_prefix"]))
    q = dev_bf16(np.concatenate([c["q"] for c in cases]))
    k = dev_bf16(np.concatenate([c["k"] for c in cases]))
    v = dev_bf16(np.concatenate([c["v"] for c in cases]))
    out_b = host_f64_of_bf16(st_b.extend_attn_batched([0, 1, 2, 3], ms, 0, q, k, v))
    row = 0
    for i in range(4):
        c = cases[i]
        single = host_f64_of_bf16(st_s.extend_attn(i, 0, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                                   dev_bf16(c["v"])))
        want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                                np.concatenate([c["v_prefix"], c["v"]]), Ps[i])
        part = out_b[row:row + ms[i]]
        assert np.abs(part - want).max() <= ATTN_TOL
        assert np.abs(part - single).max() <= ATTN_TOL
        row += ms[i]


def test_batched_split_and_unsplit_pieces_append():
    """One MFMA launch with an unsplit piece (no cached keys, one 64-key
    tile: the attention kernel appends its rows) beside split pieces (the
    combine kernel appends theirs): every piece matches the oracle and every
    appended row is in the store, bit for bit."""
    hq, hkv, d = 32, 8, 128
    Ps, ms = [0, 500, 130], [60, 30, 100]
    st = sve.KVSlots(3, 1, hq, hkv, d, 1024, 1024)
    cases = [synth.attention_case(60 + i, hq, hkv, d, Ps[i], ms[i]) for i in range(3)]
    announce("batched split and unsplit pieces")
    for i in range(3):
        toks = np.concatenate([[i + 1], np.arange(Ps[i] + ms[i] - 1)]).astype(np.int32)
        slot, r = st.kv_slot_select(toks)
        assert (slot, r) == (i, 0)
        if Ps[i]:
            st.extend_attn(slot, 0, dev_bf16(cases[i]["q_prefix"]),
                           dev_bf16(cases[i]["k_prefix"]), dev_bf16(cases[i]["v_prefix"]))
    q = dev_bf16(np.concatenate([c["q"] for c in cases]))
    k = dev_bf16(np.concatenate([c["k"] for c in cases]))
    v = dev_bf16(np.concatenate([c["v"] for c in cases]))
    out = host_f64_of_bf16(st.extend_attn_batched([0, 1, 2], ms, 0, q, k, v))
    row = 0
    for i, c in enumerate(cases):
        kc = np.concatenate([c["k_prefix"], c["k"]])
        vc = np.concatenate([c["v_prefix"], c["v"]])
        want = extend_attention(c["q"], kc, vc, Ps[i])
        assert np.abs(out[row:row + ms[i]] - want).max() <= ATTN_TOL
        kk, vv = st.kv_read(i, 0, 0, Ps[i] + ms[i])
        assert np.array_equal(host_bits(kk), kc) and np.array_equal(host_bits(vv), vc)
        row += ms[i]


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["uniform", "cached-new", "balanced"])
@pytest.mark.parametrize("case", [(28, 4, 128, 1668, 254), (28, 4, 128, 727, 134),
                                  (4, 1, 64, 1000, 90), (8, 2, 128, 64, 300),
                                  (8, 2, 128, 0, 400), (16, 16, 64, 900, 200),
                                  (32, 4, 128, 1500, 300)],
                         ids=lambda c: "h%d-%d-d%d-P%d-m%d" % c)
def test_each_split_layout_matches_oracle(case, layout):
    """The MFMA path's split tables filled each way (even tiles per split,
    cached tiles then pieces of new tiles, balanced pieces): every row
    matches the oracle and the appended rows are in the store, bit for bit.
    Full-size rows are sampled to keep the oracle fast."""
    hq, hkv, d, P, m = case
    announce(f"split layout {layout} {case}")
    c = synth.attention_case(17, hq, hkv, d, P, m)
    st = _store(hq, hkv, d, P + m + 64, max(P, m, 1))
    assert st.kv_slot_select(np.arange(P + m, dtype=np.int32)) == (0, 0)
    if P:
        st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]),
                       dev_bf16(c["v_prefix"]))
    with env(SVE_ATTN_LAYOUT=layout, SVE_MFMA_MIN_ROWS=1):
        got = host_f64_of_bf16(st.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                              dev_bf16(c["v"])))
    kc = np.concatenate([c["k_prefix"], c["k"]])
    vc = np.concatenate([c["v_prefix"], c["v"]])
    rows = np.unique(np.concatenate([np.arange(0, m, max(1, m // 40)), [m - 1]]))
    want = np.stack([extend_attention(c["q"][i:i + 1], kc[:P + i + 1], vc[:P + i + 1], P + i)[0]
                     for i in rows])
    assert np.abs(got[rows] - want).max() <= ATTN_TOL
    kk, vv = st.kv_read(0, 0, 0, P + m)
    assert np.array_equal(host_bits(kk), kc) and np.array_equal(host_bits(vv), vc)


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["uniform", "cached-new", "balanced"])
def test_each_split_layout_batched(layout):
    """Several pieces in one launch share one choice of table filling."""
    hq, hkv, d = 32, 8, 128
    Ps, ms = [0, 500, 130], [60, 30, 100]
    st = sve.KVSlots(3, 1, hq, hkv, d, 1024, 1024)
    cases = [synth.attention_case(70 + i, hq, hkv, d, Ps[i], ms[i]) for i in range(3)]
    announce(f"batched split layout {layout}")
    for i in range(3):
        toks = np.concatenate([[i + 1], np.arange(Ps[i] + ms[i] - 1)]).astype(np.int32)
        assert st.kv_slot_select(toks) == (i, 0)
        if Ps[i]:
            st.extend_attn(i, 0, dev_bf16(cases[i]["q_prefix"]),
                           dev_bf16(cases[i]["k_prefix"]), dev_bf16(cases[i]["v_prefix"]))
    q = dev_bf16(np.concatenate([c["q"] for c in cases]))
    k = dev_bf16(np.concatenate([c["k"] for c in cases]))
    v = dev_bf16(np.concatenate([c["v"] for c in cases]))
    with env(SVE_ATTN_LAYOUT=layout):
        out = host_f64_of_bf16(st.extend_attn_batched([0, 1, 2], ms, 0, q, k, v))
    row = 0
    for i, c in enumerate(cases):
        kc = np.concatenate([c["k_prefix"], c["k"]])
        vc = np.concatenate([c["v_prefix"], c["v"]])
        want = extend_attention(c["q"], kc, vc, Ps[i])
        assert np.abs(out[row:row + ms[i]] - want).max() <= ATTN_TOL
        kk, vv = st.kv_read(i, 0, 0, Ps[i] + ms[i])
        assert np.array_equal(host_bits(kk), kc) and np.array_equal(host_bits(vv), vc)
        row += ms[i]


def test_edges_empty_pieces_full_capacity_and_max_rows():
    """A batched call whose pieces include empty ones; an extend that fills a
    slot to its capacity (the last tile full, rows up to the arena's end);
    exactly max_rows rows in one call, and one more refused."""
    hq, hkv, d, cap = 28, 4, 128, 640
    announce("edges: empty pieces, full capacity, max rows")
    Ps, ms = [200, 0, 130, 64], [0, 177, 0, 63]
    st = sve.KVSlots(4, 1, hq, hkv, d, cap, 240)
    cases = [synth.attention_case(90 + i, hq, hkv, d, Ps[i], ms[i]) for i in range(4)]
    for i in range(4):
        toks = np.concatenate([[i + 1], np.arange(Ps[i] + max(ms[i], 1) - 1)]).astype(np.int32)
        assert st.kv_slot_select(toks) == (i, 0)
        if Ps[i]:
            st.extend_attn(i, 0, dev_bf16(cases[i]["q_prefix"]), dev_bf16(cases[i]["k_prefix"]),
                           dev_bf16(cases[i]["v_prefix"]))
    q = dev_bf16(np.concatenate([c["q"] for c in cases]))
    k = dev_bf16(np.concatenate([c["k"] for c in cases]))
    v = dev_bf16(np.concatenate([c["v"] for c in cases]))
    out = host_f64_of_bf16(st.extend_attn_batched([0, 1, 2, 3], ms, 0, q, k, v))
    row = 0
    for i, c in enumerate(cases):
        if ms[i]:
            want = extend_attention(c["q"], np.concatenate([c["k_prefix"], c["k"]]),
                                    np.concatenate([c["v_prefix"], c["v"]]), Ps[i])
            assert np.abs(out[row:row + ms[i]] - want).max() <= ATTN_TOL, i
        assert st.kv_len(i, 0) == Ps[i] + ms[i]
        row += ms[i]

    # a slot filled to its capacity: 400 cached rows + 240 (= max_rows) new
    P, m = cap - 240, 240
    c = synth.attention_case(95, hq, hkv, d, P, m)
    st2 = sve.KVSlots(1, 1, hq, hkv, d, cap, 400)
    assert st2.kv_slot_select(np.arange(cap, dtype=np.int32)) == (0, 0)
    st2.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]), dev_bf16(c["v_prefix"]))
    got = host_f64_of_bf16(st2.extend_attn(0, 0, dev_bf16(c["q"]), dev_bf16(c["k"]),
                                           dev_bf16(c["v"])))
    kc = np.concatenate([c["k_prefix"], c["k"]])
    vc = np.concatenate([c["v_prefix"], c["v"]])
    want = extend_attention(c["q"], kc, vc, P)
    assert np.abs(got - want).max() <= ATTN_TOL
    kk, vv = st2.kv_read(0, 0, 0, cap)
    assert np.array_equal(host_bits(kk), kc) and np.array_equal(host_bits(vv), vc)

    # max_rows: 240 rows in one call pass (above), 241 are refused
    st3 = sve.KVSlots(1, 1, hq, hkv, d, cap, 240)
    assert st3.kv_slot_select(np.arange(300, dtype=np.int32)) == (0, 0)
    q3, k3, v3 = (dev_bf16(a) for a in synth.attention_rows(synth.rng(96), 241, hq, hkv, d))
    with pytest.raises(sve.SveError):
        st3.extend_attn(0, 0, q3, k3, v3)
    assert st3.kv_len(0, 0) == 0
    st3.extend_attn(0, 0, q3[:240], k3[:240], v3[:240])
    assert st3.kv_len(0, 0) == 240


def test_kernel_timing_records_each_call():
    """Timing events around the three kernels of each timed call: positive
    attention time, a count capped at the requested calls, state errors,
    results unchanged by timing, and 0 for an append the attention kernel
    does itself."""
    hq, hkv, d, P, m = 28, 4, 128, 600, 40
    c = synth.attention_case(11, hq, hkv, d, P, m)
    st = _store(hq, hkv, d, P + m + 64, P + m)
    st.kv_slot_select(np.arange(P + m, dtype=np.int32))
    st.extend_attn(0, 0, dev_bf16(c["q_prefix"]), dev_bf16(c["k_prefix"]), dev_bf16(c["v_prefix"]))
    q, k, v = dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"])
    announce("kernel timing")
    ref = st.extend_attn(0, 0, q, k, v)
    with pytest.raises(sve.SveError) as e:
        st.timing_read()
    assert e.value.code == -5
    st.timing_start(3)
    with pytest.raises(sve.SveError):
        st.timing_start(3)
    for _ in range(5):
        st.kv_truncate(0, P)
        assert torch.equal(st.extend_attn(0, 0, q, k, v), ref)
    t = st.timing_read()
    assert t["calls"] == 3
    assert t["attn_ms"] > 0 and t["append_ms"] == 0 and t["combine_ms"] >= 0
    with env(SVE_FUSED_APPEND=0):  # the separate append kernel
        st.timing_start(1)
        st.kv_truncate(0, P)
        st.extend_attn(0, 0, q, k, v)  # its own split plan: not bitwise ref
        t0 = st.timing_read()
    assert t0["calls"] == 1 and t0["append_ms"] > 0 and t0["attn_ms"] > 0
    assert t["attn_ms"] < 3 * 10.0  # milliseconds: a sanity bound, not a speed check
