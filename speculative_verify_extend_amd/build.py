"""Build libsve.so in-tree with hipcc for gfx950.

    python -m speculative_verify_extend_amd.build [-v]

Every source under csrc/ is compiled (in parallel) and linked into
speculative_verify_extend_amd/libsve.so. Always rebuilds.
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
ARCH = os.environ.get("SVE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.cpp", "kernels_w4.hip", "kernels_attn.hip", "kernels_slot.hip",
           "kernels_probe.hip", "kernels_verify.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
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


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    noisy = [ln for ln in r.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noisy:
        print("\n".join(noisy), file=sys.stderr)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="sve_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=min(5, len(SOURCES))) as ex:
            futs = [ex.submit(_compile, s, o, verbose) for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        out_tmp = LIB + ".tmp"
        cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking libsve.so failed:\n{r.stdout}\n{r.stderr}")
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
