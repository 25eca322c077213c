"""Pins of the oracle's element and block-scale codecs.

The oracle builds its E2M1 / E4M3 values from the bit fields and rounds by
brute-force nearest search.  These tests tie that to things outside it:
torch's float8_e4m3fn decode and rounding (a library routine), the field
counts the pages state, and tie / saturation cases derived by hand from the
format definitions (tests/golden/*_rne_cases.txt).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cases(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, code = line.split()[:2]
        out.append((np.array([int(bits, 16)], np.uint32).view(np.float32)[0], int(code, 16)))
    return out


def test_e4m3_values_match_torch_float8(oracle):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_table()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # only 0x7F / 0xFF are NaN, and the largest finite value is 448
    assert list(np.nonzero(np.isnan(ours))[0]) == [0x7F, 0xFF]
    assert np.nanmax(ours) == 448.0


def test_e2m1_fields_as_the_pages_state(oracle):
    facts = json.load(open(os.path.join(GOLDEN, "format_facts.json")))
    f = facts["e2m1_fields"]
    nbits = f["sign"] + f["exponent"] + f["mantissa"]
    assert nbits == 4
    tab = oracle.e2m1_table()
    assert tab.size == 2 ** nbits
    # the sign bit is the top bit: code c and c | 8 are negatives of each other
    assert np.array_equal(tab[8:], -tab[:8])
    assert math.copysign(1.0, tab[8]) == -1.0
    # one mantissa bit: every non-zero magnitude is a power of two or 1.5 times one
    mags = tab[1:8]
    for v in mags:
        m = v / 2.0 ** math.floor(math.log2(v))
        assert m in (1.0, 1.5)
    # increasing with the code, so the code LSB is the mantissa LSB (even code = even mantissa)
    assert np.all(np.diff(tab[:8]) > 0)


def test_e2m1_values_are_the_one_mantissa_bit_subset_of_e4m3(oracle):
    """Independent pin of the E2M1 value set through torch's E4M3 decode:
    E2M1 (2 exponent bits, bias 1, 1 mantissa bit) has normal binades
    2^0..2^2 with one mantissa bit -- the E4M3 values in [1, 6] whose lower two
    mantissa bits are zero -- and an exponent-0 (subnormal) binade holding
    only 0 and 0.5 = 2^(1-bias) * 0.1b."""
    e4 = torch.arange(128, dtype=torch.uint8)
    vals = e4.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    pick = [0.0, 0.5] + sorted(v for c, v in enumerate(vals) if 1.0 <= v <= 6.0 and (c & 3) == 0)
    assert np.array_equal(oracle.e2m1_table()[:8], np.array(pick))


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_hand_derived_rounding_cases(oracle, fmt):
    cases = _cases(fmt + "_rne_cases.txt")
    v = np.array([c[0] for c in cases], np.float32)
    want = np.array([c[1] for c in cases], np.uint8)
    got = oracle.rne_sat_e2m1(v) if fmt == "e2m1" else oracle.rne_sat_e4m3(v)
    assert np.array_equal(got, want), list(zip(v, want, got))


def test_e4m3_rounding_matches_torch_in_range(oracle, synth):
    """torch's float32 -> float8_e4m3fn cast is round-to-nearest-even; below
    464 (the tie that would round to the NaN code) it agrees with RNE_SAT."""
    vals = oracle.e4m3_table()[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = []
    for m in mids:
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))]
    pts += list(vals.astype(np.float32))
    rnd = synth.uniform(7, 1, 200000) * 464.0
    pts += list(rnd.astype(np.float32))
    tiny = np.exp(synth.uniform(7, 2, 100000) * 30.0 - 26.0).astype(np.float32)   # 2^-37 .. 2^6
    pts += list(tiny)
    v = np.array(pts, np.float32)
    v = v[(v >= 0) & (v <= 464.0)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.rne_sat_e4m3(v)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(v[i], ref[i], got[i]) for i in bad[:10]]


def test_rne_sat_saturates_and_is_monotone(oracle, synth):
    v = np.sort(np.abs(synth.normal(11, 3, 100000) * 3.0).astype(np.float32))
    c2 = oracle.rne_sat_e2m1(v).astype(int)
    assert np.all(np.diff(c2) >= 0)
    v4 = np.sort(np.abs(synth.normal(11, 4, 100000) * 200.0).astype(np.float32))
    c4 = oracle.rne_sat_e4m3(v4).astype(int)
    assert np.all(np.diff(c4) >= 0)
    big = np.array([6.0001, 100.0, 3.0e38, np.inf], np.float32)
    assert np.all(oracle.rne_sat_e2m1(big) == 7)
    big4 = np.array([448.0, 470.0, 1.0e30, np.inf], np.float32)
    assert np.all(oracle.rne_sat_e4m3(big4) == 0x7E)


def test_scale_product_exact_in_16bit(oracle):
    """Every decoded unit u = s_b * e2m1(q) has at most 6 significant bits and
    lies in [2^-10, 2688], so bf16 and fp16 hold it exactly (the GEMM operand
    decode relies on this)."""
    e2 = oracle.e2m1_table()
    e4 = oracle.e4m3_table()[:0x7F]
    u = np.abs(np.outer(e4, e2)).ravel()
    u = u[u > 0]
    assert u.min() == 2.0 ** -10 and u.max() == 2688.0
    t = torch.from_numpy(u)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)
    assert torch.equal(t.to(torch.float16).to(torch.float64), t)
    # and u * 2^10 is an integer (the oracle's exact GEMM depends on it)
    assert np.all(np.floor(u * 1024.0) == u * 1024.0)
