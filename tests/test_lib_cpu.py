"""The C-ABI library loads, exports every function include/sve.h declares,
and rejects bad arguments on the host before any GPU work (CPU only)."""
import ctypes as C

import pytest

from speculative_verify_extend_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_function_is_exported(lib):
    names = _lib.header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIGS), "binding signatures cover exactly the header"


def _cfg(**kw):
    base = dict(n_slots=4, n_layers=2, n_q_heads=28, n_kv_heads=4, head_dim=128,
                capacity=2100, max_rows=256, reuse=1, match_rule=0)
    base.update(kw)
    return _lib.SveConfig(*[base[f] for f, _ in _lib.SveConfig._fields_])


def test_arena_bytes_layout(lib):
    c = _cfg()
    one = lib.sve_arena_bytes(C.byref(c), 1)
    four = lib.sve_arena_bytes(C.byref(c), 4)
    cap = 2112  # capacity rounded up to 64
    slot = 2 * (2 * 4 * cap * 128 * 2)
    assert four - one == 3 * slot
    assert one > slot


@pytest.mark.parametrize("bad", [dict(n_slots=0), dict(n_slots=5), dict(head_dim=96),
                                 dict(n_q_heads=30), dict(max_rows=0), dict(max_rows=9000),
                                 dict(n_layers=0), dict(match_rule=2),
                                 dict(capacity=1 << 20, max_rows=1 << 20)])
def test_bad_configs_are_rejected(lib, bad):
    c = _cfg(**bad)
    assert lib.sve_arena_bytes(C.byref(c), 1) == 0
    ctx, granted = C.c_void_p(), C.c_int32()
    rc = lib.sve_create(C.byref(c), C.c_void_p(256), 1 << 30, None, C.byref(ctx), C.byref(granted))
    assert rc == _lib.SVE_E_ARG


def test_create_checks_arena_before_gpu(lib):
    c = _cfg()
    ctx, granted = C.c_void_p(), C.c_int32()
    assert lib.sve_create(C.byref(c), None, 1 << 30, None, C.byref(ctx),
                          C.byref(granted)) == _lib.SVE_E_ARG
    assert lib.sve_create(C.byref(c), C.c_void_p(4096 + 16), 1 << 30, None, C.byref(ctx),
                          C.byref(granted)) == _lib.SVE_E_ARG
    assert lib.sve_create(C.byref(c), C.c_void_p(4096), 1024, None, C.byref(ctx),
                          C.byref(granted)) == _lib.SVE_E_CAPACITY
    assert b"slot" in lib.sve_last_error(None)


def test_w4_argument_checks(lib):
    assert lib.sve_w4_packed_bytes(16, 128) == 1 * 1 * (1024 + 128)
    assert lib.sve_w4_packed_bytes(17, 160) == 2 * 2 * (1024 + 128)
    assert lib.sve_w4_packed_bytes(16, 48) == 0
    p = C.c_void_p(4096)
    assert lib.sve_w4_gemv_m(p, 0, p, 16, 128, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m(p, 17, p, 16, 128, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m(p, 1, p, 16, 100, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m(None, 1, p, 16, 128, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m_routed(p, 0, 1, p, 0, p, 4, 16, 128, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m_routed(p, 2, 1, p, 1, p, 4, 16, 128, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_pack(p, p, 0, 128, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_dequant(p, 16, 31, p, None) == _lib.SVE_E_ARG
    # many-row GEMM: shape and pointer checks, and a workspace no smaller
    # than what the plan needs (all before anything is enqueued)
    assert lib.sve_w4_gemm_workspace_bytes(0, 16, 128) == 0
    assert lib.sve_w4_gemm_workspace_bytes(16, 16, 100) == 0
    assert lib.sve_w4_gemm(p, 0, p, 16, 128, p, None, 0, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemm(p, 20, p, 0, 128, p, None, 0, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemm(p, 20, p, 16, 96 + 1, p, None, 0, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemm(None, 20, p, 16, 128, p, None, 0, None) == _lib.SVE_E_ARG
    need = lib.sve_w4_gemm_workspace_bytes(254, 4608, 3584)
    assert need > 254 * 3584 * 2  # x in fp16, then a k-split plan's partials
    assert lib.sve_w4_gemm(p, 254, p, 4608, 3584, p, None, 0, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemm(p, 254, p, 4608, 3584, p, p, need - 1, None) == _lib.SVE_E_ARG


def test_null_context_is_rejected(lib):
    n = C.c_int32()
    assert lib.sve_kv_len(None, 0, 0, C.byref(n)) == _lib.SVE_E_ARG
    assert lib.sve_kv_truncate(None, 0, 0) == _lib.SVE_E_ARG
    assert lib.sve_extend_attn(None, 0, 0, None, None, None, 1, None) == _lib.SVE_E_ARG
    assert lib.sve_destroy(None) == _lib.SVE_E_ARG
    assert lib.sve_timing_start(None, 4) == _lib.SVE_E_ARG
    f, i = C.c_float(), C.c_int32()
    assert lib.sve_timing_read(None, C.byref(f), C.byref(f), C.byref(f), C.byref(i)) == _lib.SVE_E_ARG
    assert lib.sve_strerror(_lib.SVE_E_STATE) == b"call out of order"


def test_probe_arguments_fail_before_gpu_work(lib):
    """The measurement probes check their launch shapes on the host."""
    p = C.c_void_p(4096)
    ok = dict(bytes=1 << 20, blocks=256, threads=256, unroll=4, mode=0)

    def read(**kw):
        a = dict(ok, **kw)
        return lib.sve_probe_read(p, a["bytes"], a["blocks"], a["threads"], a["unroll"], a["mode"],
                                  p, None)

    assert read(bytes=0) == _lib.SVE_E_ARG
    assert read(bytes=1000) == _lib.SVE_E_ARG
    assert read(blocks=0) == _lib.SVE_E_ARG
    assert read(threads=100) == _lib.SVE_E_ARG
    assert read(threads=2048) == _lib.SVE_E_ARG
    assert read(unroll=3) == _lib.SVE_E_ARG
    assert read(mode=4) == _lib.SVE_E_ARG
    assert read(mode=3, bytes=(1 << 20) + 1024) == _lib.SVE_E_ARG     # not whole 32 KB tiles
    assert read(mode=3, threads=512) == _lib.SVE_E_ARG                # 32 KB of LDS per wave
    assert read(mode=2, bytes=(1 << 20) + 16) == _lib.SVE_E_ARG       # not whole 1 KB chunks
    assert read(mode=2, threads=1024, unroll=16) == _lib.SVE_E_ARG    # 256 KB ring > 160 KB of LDS
    assert lib.sve_probe_compute(5, 1, 1, p, None) == _lib.SVE_E_ARG
    assert lib.sve_probe_compute(0, 0, 1, p, None) == _lib.SVE_E_ARG
    assert lib.sve_probe_compute(0, 1, 0, p, None) == _lib.SVE_E_ARG
    assert lib.sve_probe_compute(0, 1, 1, None, None) == _lib.SVE_E_ARG


def test_gemv_shape_bounds_fail_before_gpu_work(lib):
    """K beyond the 32-bit activation offsets, m out of range and bad K are
    refused on the host."""
    p = C.c_void_p(4096)
    big = (1 << 22) + 32
    assert lib.sve_w4_gemv_m(p, 1, p, 16, big, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m(p, 17, p, 16, 64, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m(p, 1, p, 16, 48, p, None) == _lib.SVE_E_ARG
    assert lib.sve_w4_gemv_m_routed(p, 0, 1, p, 8, p, 4, 16, big, p, None) == _lib.SVE_E_ARG
