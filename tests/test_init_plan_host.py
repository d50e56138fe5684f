"""The summary init's split plan (near and far splits, the workspace bound),
checked on the host by tests/init_plan_check.cpp over ~520K (shape, prefix
length) pairs: exact coverage of the prefix rows, far rows at least the near
distance back, split sizes, and a workspace bound that grows with the prefix.
No GPU: the check calls host code of csrc/common.hpp only."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_init_plan_covers_the_prefix_and_fits_the_workspace(tmp_path):
    exe = str(tmp_path / "init_plan_check")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Wno-unused-command-line-argument", os.path.join(ROOT, "tests", "init_plan_check.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and " 0 failures" in r.stdout, r.stdout[-3000:]
