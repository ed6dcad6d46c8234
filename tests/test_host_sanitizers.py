"""The host layer (argument checks, workspace layout, launch set-up) built
with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only,
and the C ABI tests (tests/test_abi.py: no kernel launch, no GPU needed) run
against that build in a child process with the sanitizer runtime preloaded;
any report fails the child."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    from rejection_sampling_verifier_spec_amd.build import build_library

    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no AddressSanitizer runtime in the ROCm toolchain")
    lib = build_library(out=str(tmp_path / "libspecverify_san.so"), sanitize=True)
    env = dict(os.environ, SPECVERIFY_LIB=lib, LD_PRELOAD=rt[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
