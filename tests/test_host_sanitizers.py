"""Host code of the library under the address and undefined-behaviour
sanitizers, on the CPU: the pure host logic (configuration checks, buffer
layout, statistics, worst-case page accounting against a brute-force replay)
as a standalone program built with g++, and every C-ABI entry point's host
path in a sanitizer build of libdms loaded into a Python process with the
sanitizer runtime preloaded."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "learned_kv_cache_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_host_logic_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "host_checks")
    subprocess.run([cxx, "-std=c++17", *SAN, f"-I{ROOT}/include", f"-I{CSRC}",
                    os.path.join(HOST, "host_checks.cpp"), "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host checks ok" in r.stdout, r.stderr[-3000:]


def test_abi_host_paths_under_sanitizers():
    from learned_kv_cache_amd import build
    lib = build.SAN_OUT
    if build.sanitized_stale():
        lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(HOST, "abi_under_sanitizers.py"), lib], capture_output=True,
                       text=True, env=env, timeout=600)
    assert r.returncode == 0 and "abi checks ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
