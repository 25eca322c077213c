"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only), run against its codec, quantizer, GEMM, routing and
dequantize pins in a child process: any out-of-bounds access, use of freed
memory or undefined operation (signed overflow, bad shift, misaligned load)
aborts the run.  No GPU code is involved.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_codec.py", "test_oracle_quantize.py", "test_oracle_gemm.py",
        "test_oracle_route.py", "test_oracle_dequant.py", "test_oracle_mxfp8.py",
        "test_oracle_swiglu.py"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(src=oracle.SOURCE, path=str(tmp_path / "liboracle_san.so"), extra_flags=SAN_FLAGS)
    env = dict(os.environ, NVFP4_ORACLE_LIB=lib, LD_PRELOAD=asan,
               # the Python interpreter itself is not instrumented: its own
               # allocations are not leaks of the oracle
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(ROOT, "tests", f) for f in PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
