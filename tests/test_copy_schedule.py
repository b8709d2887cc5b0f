"""The tiled and wide GEMMs' copy waves wait with counts computed in closed
form from their fixed issue order (tiled_count.h, wide_count.h); a count that
is too large would let a barrier pass before its stage has landed, silently.
A host program replays the issue sequences for every ring shape the kernels
instantiate and compares (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "block_scaled_precision_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_copy_counts_match_replay(tmp_path):
    exe = tmp_path / "copy_schedule_check"
    src = os.path.join(ROOT, "tests", "copy_schedule_check.cpp")
    subprocess.run([HIPCC, "-O1", "-x", "hip", "--offload-arch=gfx950", "-I", CSRC, src, "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
