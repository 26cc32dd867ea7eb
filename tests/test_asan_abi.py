"""The library's host code under AddressSanitizer (CPU only).

Builds a copy of libkvfuse whose host code is ASan-instrumented (device code
unchanged) and runs tests/asan_abi_driver.c against it: every entry point's
validation path, the workspace-size and budget arithmetic, and the host
count of the static rules (checked against a brute-force count).  On a
machine without a GPU the driver also makes one valid call whose launch must
fail, with KVF_SYNC_CHECK=1 so the failure goes through the synchronising
check.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "asan_abi_driver.c")


def _has_gpu() -> bool:
    return os.path.exists("/dev/kfd")


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_host_code_under_asan(tmp_path):
    from rag_kv_cache_kvf_amd.csrc import build
    exe = build.build_asan(DRIVER)
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit: leak reports are noise here
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["KVF_SYNC_CHECK"] = "1"
    env["KVF_ASAN_LAUNCH"] = "0" if _has_gpu() else "1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    print(r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert r.returncode == 0, "driver checks failed"
    assert "all checks passed" in r.stdout
