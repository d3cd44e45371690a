"""The boundary is a C ABI: a C99 program that includes only include/cpattn.h
builds with gcc -std=c99 -pedantic -Werror, links against libcpattn.so and
gets the same host-side answers as the oracle's index code (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "context_attention_varlen_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_c_client_builds_links_and_runs(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libcpattn.so")):
        pytest.skip("libcpattn.so not built")
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, "-L", LIB_DIR, "-lcpattn",
           f"-Wl,-rpath,{LIB_DIR}"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert "c abi ok" in run.stdout
