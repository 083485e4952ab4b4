"""The host block manager under AddressSanitizer and UBSan (no GPU).

tests/block_manager_fuzz.cpp drives csrc/pool.cpp with random valid and
invalid call sequences; it is compiled here with g++ (host code only, no HIP
device code involved) and must finish without a sanitizer report, an
invariant failure or a lost block.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_block_manager_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "block_manager_fuzz"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{ROOT}/paged_kv_cache_450_amd/csrc",
           "-I/opt/rocm/include", "-o", str(exe), f"{ROOT}/tests/block_manager_fuzz.cpp",
           f"{ROOT}/paged_kv_cache_450_amd/csrc/pool.cpp"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe), "20000"], capture_output=True, text=True, env=env,
                         timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), \
        (run.stdout[-1000:], run.stderr[-3000:])
