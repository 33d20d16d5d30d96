"""ctypes loader for libsve.so (the C ABI in include/sve.h).

The library must have been built in-tree (``python -m
speculative_verify_extend_amd.build``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# SVE_LIBRARY selects another in-tree build of the same sources (the host
# sanitizer build, libsve_hostsan.so, for the CPU tests of the C ABI)
LIB_PATH = os.path.join(HERE, os.path.basename(os.environ.get("SVE_LIBRARY", "libsve.so")))
HEADER = os.path.join(os.path.dirname(HERE), "include", "sve.h")

SVE_OK = 0
SVE_E_ARG = -1
SVE_E_SLOT = -2
SVE_E_CAPACITY = -3
SVE_E_HIP = -4
SVE_E_STATE = -5
SVE_MAX_SLOTS = 4


class SveConfig(C.Structure):
    _fields_ = [
        ("n_slots", C.c_int32),
        ("n_layers", C.c_int32),
        ("n_q_heads", C.c_int32),
        ("n_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("capacity", C.c_int32),
        ("max_rows", C.c_int32),
        ("reuse", C.c_int32),
        ("match_rule", C.c_int32),
    ]


SVE_VERIFY_MAX_ROWS = 16
SVE_VERIFY_NOALLOC_MAX_V = 1 << 20
SVE_GATE_MAX_WINDOW = 64


class SpecGate(C.Structure):
    _fields_ = [
        ("k", C.c_int32),
        ("window", C.c_int32),
        ("min_accept", C.c_double),
        ("steps", C.c_int32),
        ("accepted", C.c_int32 * SVE_GATE_MAX_WINDOW),
    ]


_P = C.c_void_p
_I = C.c_int32
_SIGS = {
    "sve_arena_bytes": (C.c_size_t, [C.POINTER(SveConfig), _I]),
    "sve_create": (C.c_int, [C.POINTER(SveConfig), _P, C.c_size_t, _P, C.POINTER(_P),
                             C.POINTER(_I)]),
    "sve_destroy": (C.c_int, [_P]),
    "sve_set_stream": (C.c_int, [_P, _P]),
    "sve_info": (C.c_int, [_P, C.POINTER(_I), C.POINTER(_I)]),
    "sve_kv_slot_select": (C.c_int, [_P, _P, _I, C.POINTER(_I), C.POINTER(_I)]),
    "sve_kv_truncate": (C.c_int, [_P, _I, _I]),
    "sve_kv_len": (C.c_int, [_P, _I, _I, C.POINTER(_I)]),
    "sve_extend_attn": (C.c_int, [_P, _I, _I, _P, _P, _P, _I, _P]),
    "sve_extend_attn_batched": (C.c_int, [_P, _I, _P, _P, _I, _P, _P, _P, _P]),
    "sve_kv_read": (C.c_int, [_P, _I, _I, _I, _I, _P, _P]),
    "sve_extend_attn_questions": (C.c_int, [_P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "sve_w4_packed_bytes": (C.c_size_t, [_I, _I]),
    "sve_w4_pack": (C.c_int, [_P, _P, _I, _I, _P, _P]),
    "sve_w4_dequant": (C.c_int, [_P, _I, _I, _P, _P]),
    "sve_w4_gemv_m": (C.c_int, [_P, _I, _P, _I, _I, _P, _P]),
    "sve_w4_gemv_m_routed": (C.c_int, [_P, _I, _I, _P, _I, _P, _I, _I, _I, _P, _P]),
    "sve_w4_gemm_workspace_bytes": (C.c_size_t, [_I, _I, _I]),
    "sve_w4_gemm": (C.c_int, [_P, _I, _P, _I, _I, _P, _P, C.c_size_t, _P]),
    "sve_probe_read": (C.c_int, [_P, C.c_size_t, _I, _I, _I, _I, _P, _P]),
    "sve_probe_compute": (C.c_int, [_I, _I, _I, _P, _P]),
    "sve_probe_copy": (C.c_int, [_P, _P, C.c_size_t, _I, _P]),
    "sve_timing_start": (C.c_int, [_P, _I]),
    "sve_timing_read": (C.c_int, [_P, C.POINTER(C.c_float), C.POINTER(C.c_float),
                                  C.POINTER(C.c_float), C.POINTER(_I)]),
    "sve_verify_workspace_bytes": (C.c_size_t, [_I, _I]),
    "sve_ngram_draft": (C.c_int, [_P, _I, _I, _I, _I, _P, C.POINTER(_I)]),
    "sve_verify_accept": (C.c_int, [_P, _I, _I, _P, _P, _P, C.c_size_t, _P]),
    "sve_verify_accept_noalloc": (C.c_int, [_P, _I, _I, _P, _P, _P]),
    "sve_spec_gate_init": (C.c_int, [_P, _I, C.c_double, _I]),
    "sve_spec_gate_step": (C.c_int, [_P, _I, C.POINTER(_I)]),
    "sve_spec_break_even": (C.c_double, [C.c_double, C.c_double, _I]),
    "sve_strerror": (C.c_char_p, [C.c_int]),
    "sve_last_error": (C.c_char_p, [_P]),
}

_lib = None


def header_functions() -> list[str]:
    """Names of the functions declared in include/sve.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sve_[a-z0-9_]+)\s*\(", text)))


def load() -> C.CDLL:
    """Load libsve.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m speculative_verify_extend_amd.build` "
            "(there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class SveError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def check(code: int, ctx=None) -> None:
    if code != SVE_OK:
        lib = load()
        detail = lib.sve_last_error(ctx)
        detail = detail.decode() if detail else ""
        base = lib.sve_strerror(code).decode()
        raise SveError(code, f"{base}: {detail}" if detail else base)
