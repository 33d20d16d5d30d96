"""The library's host-side gate and break-even acceptance against the oracle
(thinkspread, 'The economics of speculative decoding', 'Gating: enable it only
where it pays' and 'Closing the ledger'), plus argument checks of the verify
entry point that fail before any GPU work (CPU only)."""
import ctypes as C

import numpy as np
import pytest

import speculative_verify_extend_amd as sve
from speculative_verify_extend_amd import _lib
from oracle.verify import RollingGate, break_even_acceptance


@pytest.mark.parametrize("seed", range(8))
def test_gate_matches_oracle_on_random_runs(seed):
    g = np.random.default_rng(seed)
    k = int(g.integers(1, 8))
    window = int(g.integers(1, 12))
    thr = float(g.choice([0.0, 0.3, 0.5, 0.6, 0.75, 1.0]))
    lib_gate, ora = sve.SpecGate(k, thr, window), RollingGate(k, thr, window)
    p = g.uniform(0.2, 1.0)
    for _ in range(60):
        acc = int(g.binomial(ora.k or k, p)) if ora.k else 0
        assert lib_gate.step(acc) == ora.step(acc)


def test_gate_boundary_is_exact():
    # rolling mean exactly at the threshold stays open in both
    for k, counts, thr in ((5, [3], 0.6), (4, [2, 3, 2], 7 / 12), (3, [1, 2], 0.5)):
        lg, og = sve.SpecGate(k, thr, 8), RollingGate(k, thr, 8)
        assert [lg.step(c) for c in counts] == [og.step(c) for c in counts]


@pytest.mark.parametrize("k", range(0, 8))
@pytest.mark.parametrize("ab", [(9.0, 5.5), (1.0, 0.0), (0.0, 1.0), (3.0, 0.7), (1.0, 100.0)])
def test_break_even_matches_oracle(k, ab):
    a, b = ab
    assert sve.spec_break_even(a, b, k) == pytest.approx(break_even_acceptance(a, b, k),
                                                         abs=1e-12)


def test_bad_gate_and_verify_arguments():
    lib = _lib.load()
    g = _lib.SpecGate()
    assert lib.sve_spec_gate_init(C.byref(g), 16, 0.6, 8) == _lib.SVE_E_ARG
    assert lib.sve_spec_gate_init(C.byref(g), 3, 1.5, 8) == _lib.SVE_E_ARG
    assert lib.sve_spec_gate_init(C.byref(g), 3, 0.6, 0) == _lib.SVE_E_ARG
    assert lib.sve_spec_gate_init(C.byref(g), 3, 0.6, 65) == _lib.SVE_E_ARG
    assert lib.sve_spec_gate_init(C.byref(g), 3, 0.6, 4) == _lib.SVE_OK
    kn = C.c_int32()
    assert lib.sve_spec_gate_step(C.byref(g), 4, C.byref(kn)) == _lib.SVE_E_ARG
    assert lib.sve_spec_gate_step(C.byref(g), -1, C.byref(kn)) == _lib.SVE_E_ARG
    assert lib.sve_spec_break_even(1.0, -1.0, 3) == -1.0
    assert lib.sve_spec_break_even(0.0, 0.0, 3) == -1.0
    assert lib.sve_verify_workspace_bytes(0, 100) == 0
    assert lib.sve_verify_workspace_bytes(17, 100) == 0
    assert lib.sve_verify_workspace_bytes(4, 151936) >= 2 * 4 * 38 * 4
    p = C.c_void_p(256)
    ws = lib.sve_verify_workspace_bytes(4, 1000)
    assert lib.sve_verify_accept(p, 0, 1000, p, p, p, ws, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept(p, 4, 0, p, p, p, ws, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept(p, 4, 1000, None, p, p, ws, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept(p, 4, 1000, p, p, p, ws - 1, None) == _lib.SVE_E_ARG


def test_noalloc_verify_arguments_fail_before_gpu_work():
    """The allocation-free verify form rejects sizes beyond its static scratch
    (and the usual bad arguments) on the host, before any HIP call."""
    lib = _lib.load()
    p = C.c_void_p(256)
    vmax = _lib.SVE_VERIFY_NOALLOC_MAX_V
    assert lib.sve_verify_accept_noalloc(p, 4, vmax + 1, p, p, None) == _lib.SVE_E_ARG
    assert b"static scratch" in lib.sve_last_error(None)
    assert lib.sve_verify_accept_noalloc(p, 0, 100, p, p, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept_noalloc(p, 17, 100, p, p, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept_noalloc(p, 4, 0, p, p, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept_noalloc(None, 4, 100, p, p, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept_noalloc(p, 4, 100, None, p, None) == _lib.SVE_E_ARG
    assert lib.sve_verify_accept_noalloc(p, 4, 100, p, None, None) == _lib.SVE_E_ARG
    # the largest vocabulary fits the scratch of the largest row count
    assert lib.sve_verify_workspace_bytes(16, vmax) <= 32768
