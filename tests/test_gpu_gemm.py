"""GPU parity of the many-row int4 GEMM against the oracle's plain product
(the same definition as the m-row GEMV, for a prefill's rows): relative L2
per row within 1e-3 (the GEMM multiplies fp16 operands: weights rounded once
to fp16, which one-hot probes read back exactly), k splits, ragged shapes,
determinism, agreement with the GEMV, and the 7B-like layer matrices at the
254 rows of the agent-turn replay's turn 9, checked on sampled columns."""
import numpy as np
import pytest
import torch

import speculative_verify_extend_amd as sve
import synth
from oracle import w4 as ow4
from tests.gpu_helpers import (announce, dev_bf16, dev_f16, dev_u8, env, rel_l2_rows,
                               require_gpu)

pytestmark = pytest.mark.gpu
GEMM_TOL = 1e-3  # relative L2 per output row


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _weights(seed, n, k):
    g = synth.rng(seed, n, k)
    w, s = synth.w4_weights(g, n, k)
    return w, s, sve.w4_pack(dev_u8(w), dev_f16(s), n, k)


@pytest.mark.parametrize("m", [16, 17, 63, 64, 65, 200, 256, 257, 300])
@pytest.mark.parametrize("n,k", [(64, 128), (100, 96), (200, 416), (1000, 160)])
def test_gemm_matches_oracle(m, n, k):
    announce(f"gemm m={m} n={n} k={k}")
    w, s, packed = _weights(20, n, k)
    x = synth.normal_bf16(synth.rng(21, m, n, k), (m, k))
    y = sve.w4_gemm(dev_bf16(x), packed, n, k).cpu().numpy()
    err = rel_l2_rows(y, ow4.gemv(x, w, s, k))
    assert err.max() <= GEMM_TOL, err


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 16])
def test_gemm_k_splits(splits):
    """Forced k splits (partials in the workspace, added in split order) all
    match the oracle, and each plan is bitwise repeatable."""
    m, n, k = 70, 300, 2048
    announce(f"gemm splits={splits}")
    w, s, packed = _weights(22, n, k)
    x = synth.normal_bf16(synth.rng(23), (m, k))
    with env(SVE_GEMM_SPLITS=splits):
        y1 = sve.w4_gemm(dev_bf16(x), packed, n, k)
        y2 = sve.w4_gemm(dev_bf16(x), packed, n, k)
    assert torch.equal(y1, y2)
    err = rel_l2_rows(y1.cpu().numpy(), ow4.gemv(x, w, s, k))
    assert err.max() <= GEMM_TOL, err


def test_gemm_one_hot_reads_the_fp16_weights():
    """x = e_c reads column c of the weights as the GEMM multiplies them:
    (code - 8) * scale rounded once to fp16, for more rows than the GEMV
    takes and across a k split."""
    n, k = 300, 1024
    w, s, packed = _weights(24, n, k)
    codes = ow4.nibbles(w, k) - 8
    scale = np.repeat(np.asarray(s, np.uint16).view(np.float16), 32, axis=1)
    dq = (codes.astype(np.float16) * scale).astype(np.float64)  # one fp16 rounding
    cols = [0, 1, 7, 8, 31, 32, 127, 128, 129, 300, 511, 512, 700, 1000, 1023, 5, 64, 96, 255,
            256]
    x = np.zeros((len(cols), k), np.float32)
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    announce("gemm one-hot")
    for splits in (1, 4):
        with env(SVE_GEMM_SPLITS=splits):
            y = sve.w4_gemm(dev_bf16(synth.f32_to_bf16_bits(x)), packed, n, k).cpu().numpy()
        for r, c in enumerate(cols):
            assert np.array_equal(y[r].astype(np.float64), dq[:, c])


def test_gemm_zero_input_and_code8():
    n, k = 64, 256
    announce("gemm zero")
    w, s, packed = _weights(25, n, k)
    y = sve.w4_gemm(torch.zeros((40, k), dtype=torch.bfloat16, device="cuda"), packed, n, k)
    assert torch.count_nonzero(y).item() == 0
    # code 8 everywhere: every weight is exactly 0
    w8 = synth.pack_nibbles(np.full((n, k), 8))
    p8 = sve.w4_pack(dev_u8(w8), dev_f16(s), n, k)
    x = dev_bf16(synth.normal_bf16(synth.rng(26), (40, k)))
    assert torch.count_nonzero(sve.w4_gemm(x, p8, n, k)).item() == 0


def test_gemm_agrees_with_gemv_and_rows_are_independent():
    """At 16 rows the GEMM and the GEMV compute the same product (different
    summation orders, both within the bound), and a row's result does not
    depend on the other rows of the call."""
    n, k = 1024, 2048
    w, s, packed = _weights(27, n, k)
    x = synth.normal_bf16(synth.rng(28), (80, k))
    announce("gemm vs gemv")
    want = ow4.gemv(x, w, s, k)
    g16 = sve.w4_gemm(dev_bf16(x[:16]), packed, n, k).cpu().numpy()
    v16 = sve.w4_gemv_m(dev_bf16(x[:16]), packed, n, k).cpu().numpy()
    assert rel_l2_rows(g16, want[:16]).max() <= GEMM_TOL
    assert rel_l2_rows(v16, want[:16]).max() <= GEMM_TOL
    assert rel_l2_rows(g16, v16).max() <= GEMM_TOL
    full = sve.w4_gemm(dev_bf16(x), packed, n, k).cpu().numpy()
    assert np.array_equal(full[:16], g16)  # same plan: same splits, same order


def test_gemm_many_row_groups():
    """More than 256 rows: several row groups of four waves, a ragged last."""
    m, n, k = 600, 128, 256
    announce("gemm 600 rows")
    w, s, packed = _weights(29, n, k)
    x = synth.normal_bf16(synth.rng(30), (m, k))
    y = sve.w4_gemm(dev_bf16(x), packed, n, k).cpu().numpy()
    assert rel_l2_rows(y, ow4.gemv(x, w, s, k)).max() <= GEMM_TOL


def test_gemm_workspace_is_checked():
    m, n, k = 254, 4608, 3584
    need = sve.w4_gemm_workspace_bytes(m, n, k)
    assert need >= m * k * 2  # x in fp16, then the split partials
    w, s, packed = _weights(31, 64, 128)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    p = torch.empty(sve.w4_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
    with pytest.raises(sve.SveError) as e:
        sve.w4_gemm(x, p, n, k, workspace=small)
    assert e.value.code == -1


@pytest.mark.parametrize("shape", synth.layer_gemv_shapes(3584, 18944, 28, 4, 128),
                         ids=["qkv", "o", "gate_up", "down"])
def test_gemm_full_7b_layer_sampled(shape):
    """7B-like layer matrices at m = 254 (the launch the bench times); the
    oracle checks 96 sampled output columns over every row."""
    n, k = shape
    m = 254
    announce(f"gemm full n={n} k={k}")
    w, s, packed = _weights(32, n, k)
    x = synth.normal_bf16(synth.rng(33), (m, k))
    y = sve.w4_gemm(dev_bf16(x), packed, n, k).cpu().numpy()
    cols = np.unique(np.concatenate([synth.rng(34).choice(n, 90, replace=False),
                                     [0, 15, 16, 63, 64, n - 65, n - 17, n - 1]]))
    err = rel_l2_rows(y[:, cols], ow4.gemv(x, w[cols], s[cols], k))
    assert err.max() <= GEMM_TOL, err


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("m,n,k", [(16, 100, 96), (70, 1000, 2048), (254, 520, 3584),
                                   (300, 4608, 640)])
def test_gemm_forms_agree_bitwise(m, n, k, splits):
    """The two workgroup forms (256 rows x 64 columns; 64 rows x 256
    columns) multiply the same fp16 operands in the same order, so under the
    same k splits their outputs are bitwise equal; both match the oracle
    (ragged rows and columns, quads past a split, several row blocks)."""
    announce(f"gemm forms m={m} n={n} k={k} splits={splits}")
    w, s, packed = _weights(35, n, k)
    x = synth.normal_bf16(synth.rng(36, m, n, k), (m, k))
    out = {}
    for form in (0, 1):
        with env(SVE_GEMM_FORM=form, SVE_GEMM_SPLITS=splits):
            out[form] = sve.w4_gemm(dev_bf16(x), packed, n, k)
    assert torch.equal(out[0], out[1])
    err = rel_l2_rows(out[1].cpu().numpy(), ow4.gemv(x, w, s, k))
    assert err.max() <= GEMM_TOL, err
