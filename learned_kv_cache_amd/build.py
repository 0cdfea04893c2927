"""Builds libdms.so (HIP, gfx950) in-tree with hipcc.

    python -m learned_kv_cache_amd.build

Every source is compiled to an object in parallel, then linked into
``learned_kv_cache_amd/libdms.so``.  Packed fp32 instructions are disabled for
device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libdms.so")
PROBE_OUT = os.path.join(PKG, "libdms_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("DMS_OFFLOAD_ARCH", "gfx950")

SOURCES = ["dms_host.hip", "decide.hip", "append.hip", "decode_attn.hip", "prefill_attn.hip", "kvzap.hip", "train_bwd.hip"]
# machine-rate probes (HBM read, bf16 matrix cores), a library of their own
PROBE_SOURCES = ["probe.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# The prefill attention kernels take maxima of scores that are never NaN
# (finite inputs, -inf for hidden keys): without NaN semantics the compiler
# emits plain v_max instead of quieting every operand first.
EXTRA_FLAGS = {"prefill_attn.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[: len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


# A build of the library with the host code under the address and
# undefined-behaviour sanitizers (device code unoptimised: it is never run),
# for the host-side tests on a machine without a GPU; kept out of the package.
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_OUT = os.path.join(SAN_DIR, "libdms_san.so")
SAN_FLAGS = [
    f"--offload-arch={ARCH}", "-O1", "-Xarch_device", "-O0", "-g", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sanitized_stale() -> bool:
    if not os.path.exists(SAN_OUT):
        return True
    t = os.path.getmtime(SAN_OUT)
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return any(os.path.getmtime(f) > t for f in srcs)


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = SAN_OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


def asan_runtime() -> str:
    """The compiler's address-sanitizer runtime (to preload into a process
    that is not itself instrumented)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("address-sanitizer runtime not found")


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
