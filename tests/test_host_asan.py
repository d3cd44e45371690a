"""The library's host code under AddressSanitizer (CPU only).

libcpattn is rebuilt with the sanitizer on its host code only (each
-fsanitize flag behind -Xarch_host; the device code is built as usual and
never run here), and two C clients built with the same compiler's sanitizer
runtime call every host-only entry point through it: the plain C ABI check
(tests/c_abi_check.c) and a seeded stress of the index plans, pair counts,
height/width split and Dynamic-CP planner (tests/host_stress_check.c, which
checks each result against properties that hold for any input).  A memory
error in the host code stops the run with a sanitizer report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    sys.path.insert(0, os.path.join(ROOT, "context_attention_varlen_amd"))
    import build
    if not (os.path.exists(build.hipcc()) and os.path.exists(CLANG)):
        pytest.skip("hipcc or the ROCm clang is missing")
    out = tmp_path_factory.mktemp("asan")
    csrc = os.path.join(ROOT, "context_attention_varlen_amd", "csrc")
    srcs = [os.path.join(csrc, s) for s in build.SOURCES]
    cmd = ([build.hipcc()] + build.HIPCC_FLAGS + ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                                 "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                                                 "-I", csrc] + srcs + ["-o", str(out / "libcpattn.so")])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


@pytest.mark.parametrize("client,expect", [("c_abi_check.c", "c abi ok"), ("host_stress_check.c", "host stress ok")])
def test_host_entry_points_under_asan(asan_lib, client, expect):
    exe = str(asan_lib / client.replace(".c", ""))
    cmd = [CLANG, "-std=c99", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", client), "-o", exe, "-L", str(asan_lib), "-lcpattn",
           f"-Wl,-rpath,{asan_lib}"]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")   # the HIP runtime keeps its allocations
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "AddressSanitizer" not in run.stderr
    assert expect in run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_stress_client_against_the_built_library(tmp_path):
    """The same stress client, plain gcc -std=c99 -pedantic -Werror, against
    the in-tree library."""
    lib_dir = os.path.join(ROOT, "context_attention_varlen_amd")
    if not os.path.exists(os.path.join(lib_dir, "libcpattn.so")):
        pytest.skip("libcpattn.so not built")
    exe = str(tmp_path / "host_stress_check")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_stress_check.c"), "-o", exe, "-L", lib_dir, "-lcpattn",
           f"-Wl,-rpath,{lib_dir}"]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr
    assert "host stress ok" in run.stdout
