"""Mutation tests of the oracle's pins (CPU only).

Each case rebuilds the oracle with one deliberate, plausible mistake planted
(`-DORACLE_MUTANT=k`, see the MUT(k) sites in oracle/nvfp4_oracle.c) and runs
the oracle's pin tests against that build in a child process: every mutant
must make at least one pin fail.  The unmutated oracle passes the same pins
in the main run.  No GPU code is involved.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    1: "outer-scale divisor 2048 instead of 6 * 448",
    2: "RNE_SAT ties go to the larger code, not the even one",
    3: "E4M3 exponent bias 8 instead of 7",
    4: "sign bit of negative elements dropped",
    5: "nibble order swapped (element 2i in the high nibble)",
    6: "block scale from a_b / (4 S) instead of a_b / (6 S)",
    7: "element divisor S instead of S * s_b",
    8: "GEMM ignores the weight's outer scale",
    9: "GEMM reads B's nibbles in the wrong order",
    10: "grouped GEMM ignores row_index",
    11: "routing ties go to the higher expert id",
    12: "SwiGLU uses sigmoid(-g)",
    13: "SwiGLU swaps the gate and up halves",
    14: "bf16 dequantization rounds twice (via fp32)",
    15: "MXFP8 scale rounded down instead of up",
    16: "fp32 -> bf16 ties away from zero",
    17: "E2M1 subnormal code m decoded as m instead of m / 2",
    18: "MXFP8 elements lose their sign",
    19: "row amax skips the last block",
    20: "dequantize indexes the outer scale by r % rows_per_scale",
}

PIN_FILES = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py")
                   and f != "test_oracle_mutants.py")


@pytest.mark.parametrize("k", sorted(MUTANTS), ids=lambda k: "M%d" % k)
def test_pins_catch_mutant(k, tmp_path):
    lib = oracle.build(mutant=k, path=str(tmp_path / ("liboracle_mut%d.so" % k)))
    env = dict(os.environ, NVFP4_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant %d (%s) survived the oracle's pins:\n%s" % (
        k, MUTANTS[k], r.stdout[-2000:])
