"""The host-side C-ABI tests again, on the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (fixed_cost_drafter_amd.sanitize).

Validation, status codes and argument marshalling run on the host only, so
this needs no GPU: the sanitized library is loaded into a child pytest with
the clang ASan runtime preloaded, and any sanitizer report fails the run.
"""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="host-side sanitizer run is for machines without a GPU")
def test_abi_host_tests_pass_under_asan_and_ubsan(tmp_path):
    from fixed_cost_drafter_amd import sanitize
    rt = sanitize.asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    lib = sanitize.build()
    env = dict(os.environ, LD_PRELOAD=rt, LONGSPARK_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:4000])
    assert " passed" in r.stdout
