"""The C ABI's host code (descriptor validation, workspace planning, the
entry points' argument checks) under AddressSanitizer and
UndefinedBehaviorSanitizer: every library source is compiled host-only with
both sanitizers, linked with tests/host_checks.cpp, and run on the CPU.  The
driver checks the statuses; the sanitizers abort on any memory error or
undefined behaviour (signed overflow in the workspace plan included)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    return os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                       else shutil.which("hipcc"))


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_host_code_under_asan_and_ubsan(tmp_path):
    from quantized_moe_expert_02_amd import build as B
    exe = B.build_host_sanitized(os.path.join(HERE, "host_checks.cpp"), str(tmp_path))
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""   # host paths only, also on a machine with a GPU
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks passed" in r.stdout
