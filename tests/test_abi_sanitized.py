"""The C ABI's host-side validation and workspace planning built with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only: GPU code is
not instrumented), and tests/test_abi.py run against that build in a child
process. Any sanitizer report aborts the child. CPU only: no call here
reaches a device.

Page: vLLM ep_fused_moe_patch.py, _ep_init -- the divisibility and range
checks the validation mirrors must reject bad arguments without touching
memory they do not own.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no ASan runtime in this ROCm toolchain")
    sys.path.insert(0, ROOT)
    from moe_expert_dispatch_amd import build
    lib = build.build_sanitized(str(tmp_path / "san"))
    env = dict(os.environ, LD_PRELOAD=rt[-1], MOE_HIP_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in r.stdout
