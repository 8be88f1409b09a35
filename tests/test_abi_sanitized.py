"""Host-only: the C-ABI layer (kvd_api.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer against recording stubs of its device side (tests/host_abi), then
driven through every entry point: each documented error path, and a seeded sweep of edge-value
dims whose accepted calls must launch inside what the kernels assume.  No GPU is needed; g++
builds host code only, with the HIP headers for the runtime's types."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_abi")
API = os.path.join(ROOT, "quantized_kv_cache_split_amd", "csrc", "kvd_api.cpp")
ROCM_INCLUDE = "/opt/rocm/include"


def _sanitized_binary(tmp):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    flags = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
             "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "quantized_kv_cache_split_amd", "csrc"), "-I", HERE,
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g", "-O1", "-Wall", "-Wextra", "-Werror"]
    objs = []
    for src in (API, os.path.join(HERE, "launch_stub.cpp"), os.path.join(HERE, "abi_sweep.cpp")):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        res = subprocess.run([gxx, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        objs.append(obj)
    exe = os.path.join(tmp, "abi_sweep")
    res = subprocess.run([gxx, "-fsanitize=address,undefined", *objs, "-o", exe],
                         capture_output=True, text=True)
    if res.returncode != 0 and "asan" in res.stderr:
        pytest.skip("sanitizer runtime libraries are not installed")
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def sweep_exe(tmp_path_factory):
    return _sanitized_binary(str(tmp_path_factory.mktemp("abi_san")))


@pytest.mark.parametrize("seed", [1, 20260101])
def test_c_abi_under_asan_ubsan(sweep_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sweep_exe, "150000", str(seed)], capture_output=True, text=True,
                         env=env, timeout=600)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "all checks passed" in res.stdout
    assert int(res.stdout.split("skewed runs ")[1].split(",")[0]) > 0, res.stdout
    assert int(res.stdout.split("early-skewed ")[1].split(",")[0]) > 0, res.stdout
    assert int(res.stdout.split("one-block ")[1].split()[0]) > 0, res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
