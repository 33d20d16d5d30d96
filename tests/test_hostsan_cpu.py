"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU tests of the library (argument checks,
the host-only gate, break-even and n-gram drafting) run in a child process
against libsve_hostsan.so, the same sources with api.cpp built with both
sanitizers (host code only), the sanitizer runtime preloaded. Any report
fails the child and so this test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOSTSAN = os.path.join(ROOT, "speculative_verify_extend_amd", "libsve_hostsan.so")
CPU_ABI_TESTS = ["tests/test_lib_cpu.py", "tests/test_verify_host.py", "tests/test_ngram_host.py"]


def _asan_runtime():
    for pat in ("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def test_c_abi_cpu_tests_under_host_sanitizers():
    if not os.path.exists(HOSTSAN):
        pytest.skip("libsve_hostsan.so is not built (python -m speculative_verify_extend_amd.build)")
    # the C ABI really is instrumented (and the ordinary build is not)
    import shutil
    if shutil.which("nm"):
        und = subprocess.run(["nm", "-D", "--undefined-only", HOSTSAN], capture_output=True,
                             text=True).stdout
        assert "__asan_" in und and "__ubsan_" in und
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm")
    env = dict(os.environ, LD_PRELOAD=rt, SVE_LIBRARY="libsve_hostsan.so",
               ASAN_OPTIONS="detect_leaks=0:exitcode=66",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run(
        [sys.executable, "-c", "from speculative_verify_extend_amd import _lib; print(_lib.load()._name)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip().endswith("libsve_hostsan.so")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p",
                        "no:cacheprovider", *CPU_ABI_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
