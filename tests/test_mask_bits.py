"""The kernels' mask helpers on the host: the interval forms of the mask
(per query and per key) against the position predicate, and the per-block
bit sets the attention kernels test partial tiles with against the interval
test (CPU only; built with hipcc as host code)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_attention_varlen_amd", "csrc")


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


@pytest.mark.skipif(_hipcc() is None, reason="no hipcc")
def test_mask_bit_sets_match_the_interval_test(tmp_path):
    exe = str(tmp_path / "mask_bits_check")
    cmd = [_hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(ROOT, "tests", "mask_bits_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "mask bits ok" in run.stdout
