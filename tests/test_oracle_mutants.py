"""Mutation tests of the oracle's pins (CPU only).

Each case copies oracle/nvfp4_oracle.c, plants one deliberate, plausible
mistake by replacing a snippet of the copy, builds the copy into a temporary
library and runs the oracle's pin tests against it in a child process: every
mutant must make at least one pin fail.  The unmodified oracle passes the
same pins in the main run, and its source carries no trace of the mutants.
No GPU code is involved.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# id: (what the mistake is, original snippet, planted snippet, occurrences of
# the snippet), or (what, [(original, planted), ...]) with each original
# occurring once
MUTANTS = {
    1: ("outer-scale divisor 2048 instead of 6 * 448",
        "amax / 2688.0f", "amax / 2048.0f", 2),
    2: ("RNE_SAT ties go to the larger code, not the even one",
        "(d == bestd && (c & 1) == 0)", "(d == bestd)", 1),
    3: ("E4M3 exponent bias 8 instead of 7",
        "(1.0 + m / 8.0) * ldexp(1.0, e - 7)", "(1.0 + m / 8.0) * ldexp(1.0, e - 8)", 1),
    4: ("sign bit of negative elements dropped",
        "codes[j] = (uint8_t)((signbit(xs[j]) ? 8 : 0) | mag);", "codes[j] = (uint8_t)mag;", 1),
    5: ("nibble order swapped (element 2i in the high nibble)",
        "(uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4))",
        "(uint8_t)(codes[2 * j + 1] | (codes[2 * j] << 4))", 1),
    6: ("block scale from a_b / (4 S) instead of a_b / (6 S)",
        "float t = 6.0f * S;", "float t = 4.0f * S;", 1),
    7: ("element divisor S instead of S * s_b",
        "float d = S * sbv;", "float d = S;", 1),
    8: ("GEMM ignores the weight's outer scale",
        [("* (double)b_s[b_scale[i]] *", "*"), ("* (double)b_s[0] *", "*"), ("* (double)b_s[g] *", "*")]),
    9: ("GEMM reads B's nibbles in the wrong order",
        "int cb = (j & 1) ? (bq[j / 2] >> 4) : (bq[j / 2] & 15);",
        "int cb = (j & 1) ? (bq[j / 2] & 15) : (bq[j / 2] >> 4);", 1),
    10: ("grouped GEMM ignores row_index",
         "row_index ? row_index[i] : i", "i", 1),
    11: ("routing ties go to the higher expert id",
         "lt[e] > lt[best]", "lt[e] >= lt[best]", 1),
    12: ("SwiGLU uses sigmoid(-g)",
         "(1.0 + exp(-g))", "(1.0 + exp(g))", 1),
    13: ("SwiGLU swaps the gate and up halves",
         "double g = gr[j], u = gr[f + j];", "double g = gr[f + j], u = gr[j];", 1),
    14: ("bf16 dequantization rounds twice (via fp32)",
         "out[r * k + j] = f64_to_bf16_nearest(S * sbv * oracle_e2m1_value(code));",
         "out[r * k + j] = f32_to_bf16_nearest((float)(S * sbv * oracle_e2m1_value(code)));", 1),
    15: ("MXFP8 scale rounded down instead of up",
         "while (ldexp(448.0, e) < amax) ++e;   /* smallest e with amax <= 448 * 2^e */",
         "while (ldexp(448.0, e) < amax) ++e;\n    if (e > -127) e = (int)floor(log2(amax)) - 8;", 1),
    16: ("fp32 -> bf16 ties away from zero",
         "return (lo & 1) ? hi : lo;", "return hi;", 1),
    17: ("E2M1 subnormal code m decoded as m instead of m / 2",
         "(e == 0) ? 0.5 * m :", "(e == 0) ? 1.0 * m :", 1),
    18: ("MXFP8 elements lose their sign",
         "((signbit(xv) ? 0x80 : 0) | mag)", "(0 | mag)", 1),
    19: ("row amax skips the last block",
         "row_amax(xr, k)", "row_amax(xr, k > 16 ? k - 16 : k)", 1),
    20: ("dequantize indexes the outer scale by r % rows_per_scale",
         "double S = (double)s[r / rows_per_scale];", "double S = (double)s[r % rows_per_scale];", 1),
    # the fp32 step order of the contract (a reading of the pages' real-valued
    # formula x / (S * s_b)): the literal per-element division, and a block
    # quotient formed in fp64 instead of fl32(a_b / fl32(6 S))
    21: ("element ratio x / d instead of x * fl32(1 / d)",
         "float r = xs[j] * inv;", "float r = xs[j] / d;", 1),
    22: ("block quotient a_b / (6 S) in fp64, rounded to E4M3 once",
         "sc = oracle_rne_sat_e4m3(v);",
         "sc = rne_sat_search((double)ab / (6.0 * (double)S), 128, oracle_e4m3_value); (void)v;", 1),
}

PIN_FILES = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py")
                   and f != "test_oracle_mutants.py")


def mutant_source(k):
    m = MUTANTS[k]
    edits = [(m[1], m[2], m[3])] if len(m) == 4 else [(o, n, 1) for o, n in m[1]]
    src = open(oracle.SOURCE).read()
    for old, new, count in edits:
        assert src.count(old) == count, "mutant %d: snippet found %d times, expected %d" % (
            k, src.count(old), count)
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_mutant_snippets_match_the_oracle(k):
    mutant_source(k)


@pytest.mark.parametrize("k", sorted(MUTANTS), ids=lambda k: "M%d" % k)
def test_pins_catch_mutant(k, tmp_path):
    src = tmp_path / ("nvfp4_oracle_mut%d.c" % k)
    src.write_text(mutant_source(k))
    lib = oracle.build(src=str(src), path=str(tmp_path / ("liboracle_mut%d.so" % k)))
    env = dict(os.environ, NVFP4_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant %d (%s) survived the oracle's pins:\n%s" % (
        k, MUTANTS[k][0], r.stdout[-2000:])
