"""Build libpagedkv.so for gfx950 with hipcc, in-tree.

    python paged_kv_cache_450_amd/build.py [-v]

It is run as a script (or loaded by file path) so that it does not import
the package, whose import loads the library it builds.

Objects go to <repo>/_build/, the shared library next to this file.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["pool.cpp", "prefix_plan.cpp", "append.hip", "decode.hip", "reduce.hip", "copy.hip",
           "swap.hip"]
# The gather-rate probe (a measuring instrument for bench.py, not the decode
# path) goes into a library of its own.
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libpkvprobe.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; install ROCm or put hipcc on PATH")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON_FLAGS, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(path)} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared libraries (the decode library
    and the probe library); returns the decode library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
