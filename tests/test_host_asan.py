"""The C ABI's host side under AddressSanitizer and UBSan, with no GPU.

A host-only library is built from the argument checks (api.cpp), the launch
planning (plans.cpp) and test-only launcher stand-ins
(tests/host_asan/launch_stub.cpp) with g++ -fsanitize=address,undefined.
Then, in a child process with the sanitizer runtime preloaded:
  * the whole of tests/test_abi.py runs against it (every status code,
    every size query, every symbol export);
  * a launch that fails makes each entry point return QG_ERR_HIP, with that
    one launch attempted and nothing after it (the failure of the first of
    several launches, or of the scratch lookup of the no-allocation GEMM,
    stops the call).
Any out-of-bounds access, use after free or undefined behaviour in that
host code aborts the child, and the test fails.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_group_quantized_amd", "csrc")

_CHILD = r"""
import ctypes, sys
sys.path.insert(0, %(root)r)
import int8_group_quantized_amd.binding as B
B._LIB_PATH = %(lib)r
B._lib = None
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", "--rootdir", %(root)r,
                  %(root)r + "/tests/test_abi.py"])
print("ABI_TESTS_RC", int(rc), flush=True)

L = ctypes.CDLL(%(lib)r)
P, I64, INT, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
L.qg_test_fail_launches.argtypes = [INT]
L.qg_test_launch_calls.restype = ctypes.c_long
for name, (args, res) in B._SIGNATURES.items():
    getattr(L, name).argtypes = args
    getattr(L, name).restype = res
F = 0x10000
HIP = 6
items = (B.GroupItem * 2)(B.GroupItem(F, F, F, 512), B.GroupItem(F, F, F, 1024))
calls = {
    "qgemm_w4a16 M=1": lambda: L.qgemm_w4a16(F, F, F, 1, F, 1, 2560, 19456, 0, 0, None),
    "qgemm_w4a16 M=16 split-K": lambda: L.qgemm_w4a16(F, F, F, 1, F, 16, 9728, 2560, F, 1 << 30, None),
    "qgemm_w4a16 prefill": lambda: L.qgemm_w4a16(F, F, F, 1, F, 300, 1280, 336, F, 1 << 30, None),
    "qgemm_w8f16 M=3": lambda: L.qgemm_w8f16(F, F, F, 0, F, 3, 896, 592, F, 1 << 30, None),
    "qgemm_w4a16_plan": lambda: L.qgemm_w4a16_plan(F, F, F, 1, F, 3, 1024, 64, F, 1 << 30, 1, 1, 4, None),
    "qgemm_w4a16_noalloc": lambda: L.qgemm_w4a16_noalloc(F, F, F, 1, F, 16, 9728, 2560, None),
    "qgemm_w4a16_grouped M=1": lambda: L.qgemm_w4a16_grouped(F, items, 2, 1, 1, 2560, F, 1 << 30, None),
    "qgemm_w8a16_grouped M=16": lambda: L.qgemm_w8a16_grouped(F, items, 2, 0, 16, 2560, F, 1 << 30, None),
    "qg_pack_to_grid_w4": lambda: L.qg_pack_to_grid_w4(F, 2, F, 1, 256, 512, F, None),
    "qg_rtn_scales_w8": lambda: L.qg_rtn_scales_w8(F, 0, 256, 512, F, None),
    "qg_prepack_w4": lambda: L.qg_prepack_w4(F, 256, 512, F, None),
    "qg_unpack_w8": lambda: L.qg_unpack_w8(F, 256, 512, F, None),
    "qg_dequant_w4": lambda: L.qg_dequant_w4(F, F, 1, 256, 512, F, 0, None),
    "qg_fake_quant_w8": lambda: L.qg_fake_quant_w8(F, 2, F, 0, 256, 512, F, 0, None),
    "qg_prepack_scales": lambda: L.qg_prepack_scales(F, 1, 256, 512, F, None),
    "qg_swa_attention": lambda: L.qg_swa_attention(F, F, F, F, F, 1, 16, 20, 4, 128, 8208, 1024,
                                                   0.088, F, 1 << 30, None),
    "qg_read_stream": lambda: L.qg_read_stream(F, 1 << 20, 1024, F, None),
}
bad = []
for name, fn in calls.items():
    L.qg_test_reset()
    ok_status = fn()
    ok_calls = L.qg_test_launch_calls()
    L.qg_test_reset()
    L.qg_test_fail_launches(1)
    st = fn()
    n = L.qg_test_launch_calls()
    if ok_status != 0 or ok_calls < 1 or st != HIP or n != 1:
        bad.append((name, ok_status, ok_calls, st, n))
# the no-allocation GEMM whose scratch lookup fails: QG_ERR_HIP, nothing launched
L.qg_test_reset()
L.qg_test_fail_launches(2)
st = L.qgemm_w4a16_noalloc(F, F, F, 1, F, 16, 9728, 2560, None)
if st != HIP or L.qg_test_launch_calls() != 0:
    bad.append(("noalloc scratch lookup", st, L.qg_test_launch_calls()))
print("LAUNCH_FAILURE_CASES", len(calls) + 1, "BAD", bad, flush=True)
sys.exit(int(rc) or (1 if bad else 0))
"""


def _asan_runtime():
    gxx = shutil.which("g++")
    if gxx is None:
        return None, None
    rt = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = rt.stdout.strip()
    return gxx, (path if os.path.isabs(path) and os.path.exists(path) else None)


def test_abi_checks_under_address_sanitizer(tmp_path):
    gxx, asan = _asan_runtime()
    if gxx is None or asan is None:
        pytest.skip("g++ with AddressSanitizer is not available")
    lib = str(tmp_path / "libqgemm_hostcheck.so")
    cmd = [gxx, "-std=c++17", "-shared", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plans.cpp"),
           os.path.join(ROOT, "tests", "host_asan", "launch_stub.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    child = _CHILD % {"root": ROOT, "lib": lib}
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       timeout=600, cwd=str(tmp_path))
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert "ABI_TESTS_RC 0" in out, out[-6000:]
    assert "BAD []" in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
