"""Build libsve.so in-tree with hipcc for gfx950.

    python -m speculative_verify_extend_amd.build [-v]

Every source under csrc/ is compiled (in parallel) and linked into
speculative_verify_extend_amd/libsve.so. Always rebuilds.

It also links libsve_hostsan.so: the same kernels with the host side (the C
ABI in api.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer,
host code only (no sanitizer in GPU code). The CPU tests of the C ABI run
against it in a child process that preloads the sanitizer runtime.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsve.so")
LIB_HOSTSAN = os.path.join(HERE, "libsve_hostsan.so")
# host-only sanitizers for the C ABI (each -fsanitize right after -Xarch_host)
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
ARCH = os.environ.get("SVE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.cpp", "kernels_w4.hip", "kernels_attn.hip", "kernels_slot.hip",
           "kernels_probe.hip", "kernels_verify.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # kernel arguments of scalar and pointer type start out in scalar
    # registers (the first 16 dwords), so a kernel's first loads do not wait
    # for a load of its argument block; kernels taking one parameter struct
    # by value are not eligible and load it as before
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", INCLUDE, "-I", CSRC,
]


# per-source extra flags. The compute probes keep MFMA accumulators in
# ordinary vector registers: with the default (accumulation registers) the
# compiler copies the eight 16x16 accumulators around the probe's loop, and
# the probe would time the copies instead of the matrix cores.
EXTRA_FLAGS = {"kernels_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libsve)")


def _compile(src: str, obj: str, verbose: bool, extra=()) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    noisy = [ln for ln in r.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noisy:
        print("\n".join(noisy), file=sys.stderr)


def _link(objs, out: str, verbose: bool, extra=()) -> None:
    out_tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(out_tmp, out)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="sve_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        san_api = os.path.join(tmp, "api_hostsan.o")
        with cf.ThreadPoolExecutor(max_workers=min(6, len(SOURCES) + 1)) as ex:
            futs = [ex.submit(_compile, s, o, verbose) for s, o in zip(SOURCES, objs)]
            futs.append(ex.submit(_compile, "api.cpp", san_api, verbose, HOSTSAN_FLAGS))
            for f in futs:
                f.result()
        _link(objs, LIB, verbose)
        _link([san_api] + [o for s, o in zip(SOURCES, objs) if s != "api.cpp"], LIB_HOSTSAN,
              verbose, ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-shared-libsan"])
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
