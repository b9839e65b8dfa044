"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp, tilemap_host.cpp and plan_host.cpp are built with g++
-fsanitize=address,undefined into a host-only library whose device launchers
are stubs that answer "no device" (tests/host_sanitize/launch_stubs.cpp).
The ABI, host tile-map and schedule tests then run against that library in
a child process with the ASan runtime preloaded (SVGA_LIBRARY points the
binding at it). Any sanitizer report ends the child with a nonzero status and
fails this test; the reports are written to files and shown.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_spatio_amd", "csrc")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "tilemap_host.cpp", "plan_host.cpp")]
STUBS = os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp")
CHILD_TESTS = ["tests/test_abi.py", "tests/test_tilemap_host.py", "tests/test_schedule.py"]


def build_sanitized(gxx, out):
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *HOST_SOURCES, STUBS, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("needs g++ and the HIP headers")
    libasan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("g++ has no AddressSanitizer runtime")
    lib = str(tmp_path / "libsvga_host_sanitized.so")
    build_sanitized(gxx, lib)
    logs = str(tmp_path / "report")
    env = dict(os.environ, SVGA_LIBRARY=lib, LD_PRELOAD=libasan,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}",
               UBSAN_OPTIONS=f"print_stacktrace=1:log_path={logs}")
    # the child binds the sanitized build, not libsvga.so
    probe = subprocess.run([sys.executable, "-c", "from block_sparse_spatio_amd import _lib; _lib.lib(); "
                            "print(_lib.LIB_PATH)"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *CHILD_TESTS], env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    reports = "".join(open(p).read() for p in sorted(glob.glob(logs + "*")))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-2000:] + reports[-6000:])
    assert " passed" in r.stdout
