"""The CPU oracle and the library's host-side argument validation under
AddressSanitizer and UndefinedBehaviorSanitizer.

Each runs in a subprocess with the sanitizer runtime preloaded (Python
itself is not instrumented; leak reports are off).  The oracle is rebuilt
with -fsanitize=address,undefined and runs every entry point on small
inputs; the library is rebuilt with the sanitizers on its host code only
(no GPU is touched: every call here fails validation before any launch).
Any sanitizer report, or a non-zero exit, fails the test."""
import os
import subprocess
import sys
import tempfile

import pytest

import glob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
# the library is built by hipcc (clang): its host code takes clang's runtime,
# which carries the UndefinedBehaviorSanitizer handlers as well
CLANG_RT = (glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so") + [""])[0]
ENV = dict(os.environ, LD_PRELOAD=ASAN_RT, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)

ORACLE_DRIVER = r'''
import numpy as np, oracle
from mxfp4_precision_numerics_amd import synth
oracle._LIB = LIB
rng = np.random.default_rng(0)
x = synth.channel_scaled_activations(rows=40, cols=96, seed=1)
for rht in (False, True):
    for rnd in (0, 1):
        oracle.quantize_1d(x, use_rht=rht, sign_mask=0x1234, rnd=rnd, seed=3, threads=2)
        oracle.quantize_1d(x, block_axis=0, group_offsets=[0, 7, 7, 40], use_rht=rht, sign_mask=5, rnd=rnd,
                           seed=3, threads=2)
        oracle.quantize_1d_ex(x, use_rht=rht, rnd=rnd, clip_ratio=0.0, macro_block=96, threads=2)
        oracle.quantize_1d_ex(x, use_rht=rht, rnd=rnd, clip_ratio=0.75, threads=2)
w = (rng.standard_normal((2, 64, 96)) * 0.02).astype(np.float32)
c, s, ct, st = oracle.quantize_2d(w, threads=2)
oracle.quantize_2d_deosc(w * 1.01, c, s, 9, threads=2)
oracle.dequantize(c, s, block_rows=32, threads=2)
cc, ss, mr = oracle.quantize_1d_ex(x, macro_block=32)
oracle.dequantize_1d_ex(cc, ss, mr, macro_block=32, threads=2)
ac, asc = oracle.quantize_1d(x)
oracle.grouped_gemm(ac, asc, ac[None], asc[None], [0, 40], 40, 40, 96, threads=2)
oracle.grouped_gemm(ac, asc, ac, asc, [0, 32, 96], 40, 40, 96, group_dim_k=True, threads=2)
oracle.round_bf16_bits([1.0, 3.4e38, float("nan"), -2.0 ** -134])
oracle.philox4x32_10([1, 2, 3, 4], [5, 6])
print("oracle ok")
'''


def _run(code, **env):
    r = subprocess.run([sys.executable, "-c", code], env=dict(ENV, **env), capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


@pytest.mark.skipif(not os.path.exists(ASAN_RT), reason="no AddressSanitizer runtime")
def test_oracle_under_address_and_undefined_behavior_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_asan.so")
        subprocess.check_call(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                               "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                               "-fno-omit-frame-pointer", "-o", lib, os.path.join(ROOT, "oracle", "mx_oracle.c"),
                               "-lm"])
        out = _run("LIB = %r\n" % lib + ORACLE_DRIVER)
        assert "oracle ok" in out


LIBRARY_DRIVER = r'''
import ctypes
L = ctypes.CDLL(LIB)
P, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
F = P(0x1000)
for name in ("mx_rht", "mx_quantize_1d", "mx_quantize_2d", "mx_quantize_2d_deosc", "mx_dequantize",
             "mx_grouped_gemm", "mx_grouped_gemm_q", "mx_quantize_1d_ex", "mx_dequantize_1d_ex",
             "mx_quantize_1d_dual"):
    getattr(L, name).restype = ctypes.c_int
assert L.mx_rht(F, 0, F, i64(4), i64(48), 0, 0, None) == 2
assert L.mx_quantize_1d(F, 1, i64(4), i64(33), 1, None, 0, i64(0), None, 0, 0, 0, u64(0), 0, u64(0), F, i64(0), F, None) == 2
assert L.mx_quantize_1d(F, 1, i64(4), i64(32), 0, None, 2, i64(64), None, 0, 0, 0, u64(0), 0, u64(0), F, i64(0), F, None) == 1
assert L.mx_quantize_2d(F, 1, i64(1), i64(48), i64(32), F, i64(0), F, None, i64(0), None, None) == 2
assert L.mx_quantize_2d_deosc(F, 0, i64(1), i64(64), i64(64), F, i64(0), F, 40, F, i64(0), F, None, i64(0), None, None, None) == 2
assert L.mx_dequantize(F, i64(0), None, i64(1), i64(4), i64(32), 1, F, 0, None) == 1
assert L.mx_grouped_gemm(F, i64(0), F, None, F, i64(0), F, 0, F, 0, 0, i64(64), i64(64), i64(64), ctypes.c_float(1.0), F, 1, None) == 2
assert L.mx_grouped_gemm_q(F, i64(0), F, None, F, i64(0), F, 0, F, 1, i64(64), i64(64), i64(64), ctypes.c_float(1.0), F, None, i64(0), F, None) == 1
assert L.mx_quantize_1d_ex(F, 0, i64(4), i64(256), 0, 0, 0, u64(0), 0, u64(0), ctypes.c_float(2.0), i64(0), F, F, None, None) == 2
assert L.mx_dequantize_1d_ex(F, F, None, i64(4), i64(256), i64(128), F, None) == 1
assert L.mx_quantize_1d_dual(F, 1, i64(64), i64(48), F, 2, i64(128), 1, 0, 1, 0, u64(0), F, F, 1, 0, u64(0), F, i64(0), F, u64(0), 0, None) == 2
# empty inputs return before looking at any pointer
assert L.mx_quantize_2d(None, 1, i64(0), i64(32), i64(32), None, i64(0), None, None, i64(0), None, None) == 0
assert L.mx_grouped_gemm(F, i64(0), F, None, F, i64(0), F, 0, F, 1, 0, i64(0), i64(64), i64(64), ctypes.c_float(1.0), None, 1, None) == 0
print("library ok")
'''


@pytest.mark.skipif(not os.path.exists(CLANG_RT), reason="no clang AddressSanitizer runtime")
def test_library_host_validation_under_sanitizers():
    src = os.path.join(ROOT, "mxfp4_precision_numerics_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libmx355_asan.so")
        cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-o", lib, os.path.join(src, "mx_quant.hip"), os.path.join(src, "mx_gemm.hip")]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        out = _run("LIB = %r\n" % lib + LIBRARY_DRIVER, LD_PRELOAD=CLANG_RT)
        assert "library ok" in out
