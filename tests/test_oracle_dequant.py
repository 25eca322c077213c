"""Pins for the oracle's bf16 dequantization (dequantized-backward mode,
Miles page, section 反量化反向模式) and its single rounding double -> bf16.

  - brute force: exact rational arithmetic (fractions.Fraction) picks the
    nearest bf16 on random doubles of up to 30 significant bits, on
    constructed ties, subnormals and the overflow threshold;
  - library routine: torch's conversion agrees wherever the double is an
    fp32 value (no double rounding possible there);
  - closed form: with a power-of-two outer scale the product has at most six
    significant bits, so the bf16 value equals S * s_b * e2m1 exactly;
  - brute force on dequantized entries: a sample of outputs re-derived from
    the codes with Fractions.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthgen as sg


def bf16_value(b):
    return float((np.array([b], np.uint32) << 16).view(np.float32)[0])


def nearest_bf16_fraction(x):
    """Brute force: among bf16 patterns around x, the nearest in exact
    rational arithmetic, ties to the even pattern."""
    fx = Fraction(x)
    b = int((np.array([np.float32(x)], np.float32).view(np.uint32)[0]) >> 16)
    cands = set()
    for d in range(-2, 3):
        c = (b + d) & 0xFFFF
        if (c & 0x7F80) == 0x7F80 and (c & 0x7F):
            continue  # NaN patterns
        cands.add(c)
    best = None
    for c in sorted(cands):
        v = bf16_value(c)
        dist = abs(Fraction(2) ** 128 - abs(fx)) if np.isinf(v) else abs(Fraction(v) - fx)
        if np.isinf(v) and np.sign(v) != np.sign(x):
            continue
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_f64_to_bf16_brute_force(oracle):
    rng = np.random.default_rng(1)
    n = 4000
    mant = rng.integers(1 << 29, 1 << 30, n).astype(np.float64)
    exps = rng.integers(-170, 100, n)
    x = np.ldexp(mant, exps - 29) * rng.choice([-1.0, 1.0], n)
    got = oracle.f64_to_bf16(x)
    for xi, g in zip(x, got):
        assert int(g) == nearest_bf16_fraction(float(xi)), xi


def test_f64_to_bf16_ties_subnormals_overflow(oracle):
    cases = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8) - 2.0 ** -40,
             2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** -126 * (1 + 2.0 ** -8),
             float(Fraction(2) ** 128 - Fraction(2) ** 119), float(Fraction(2) ** 128 - Fraction(2) ** 120),
             float(Fraction(2) ** 128 - Fraction(2) ** 119 - Fraction(2) ** 90), 5e-324, -0.0, 0.0]
    got = oracle.f64_to_bf16(np.array(cases))
    for xi, g in zip(cases, got):
        if xi == 0.0:
            assert int(g) == (0x8000 if np.signbit(xi) else 0)
        else:
            assert int(g) == nearest_bf16_fraction(xi), xi


def test_f64_to_bf16_matches_torch_on_fp32_values(oracle):
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, 1 << 18, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)].astype(np.float64)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(f), want)


def _quantized(oracle, rows, k, seed):
    x = sg.student_t3_bf16(seed, sg.S_X, (rows, k))
    return oracle.quantize_rows(x)


def test_dequantize_power_of_two_scale_is_exact(oracle):
    q, sb, _ = _quantized(oracle, 16, 256, 11)
    s = np.ldexp(np.ones(16, np.float32), np.arange(-20, 12, 2)).astype(np.float32)
    out = oracle.dequantize_bf16(q, sb, s)
    exact = oracle.dequantize(q, sb, s)
    vals = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(vals, exact)


def test_dequantize_entries_brute_force(oracle):
    q, sb, s = _quantized(oracle, 24, 512, 12)
    # outer scales with few significant bits make ties common
    s = (s.view(np.uint32) & np.uint32(0xFFFF8000)).view(np.float32)
    s[::3] = sg.uniform(3, 1, 8).astype(np.float32) * 1e-3
    out = oracle.dequantize_bf16(q, sb, s)
    e2m1 = oracle.e2m1_table()
    e4m3 = oracle.e4m3_table()
    rng = np.random.default_rng(4)
    for _ in range(3000):
        r, j = int(rng.integers(24)), int(rng.integers(512))
        byte = int(q[r, j // 2])
        code = (byte >> 4) if j & 1 else (byte & 15)
        x = Fraction(float(s[r])) * Fraction(float(e4m3[sb[r, j // 16]])) * Fraction(float(e2m1[code]))
        want = nearest_bf16_fraction(float(x)) if x != 0 else (0x8000 if code & 8 else 0)
        assert float(x) == x  # the product is exact in a double
        assert int(out[r, j]) == want, (r, j)


def test_dequantize_weight_scale_index(oracle):
    w = sg.normal_bf16(21, sg.S_W, (3, 40, 64), 0.0, 0.02)
    q, sb, s, _ = oracle.quantize_weight(w)
    out = oracle.dequantize_bf16(q.reshape(120, 32), sb.reshape(120, 4), s, rows_per_scale=40)
    for g in range(3):
        part = oracle.dequantize_bf16(q[g], sb[g], np.repeat(s[g], 40))
        assert np.array_equal(out[40 * g:40 * (g + 1)], part)


def fp32_tie_scales(count=64):
    """Outer scales S (fp32) for which 1.5 * S, rounded to fp32, lands exactly
    on a bf16 halfway point while the exact product does not: rounding twice
    (via fp32) and once disagree there."""
    m = np.arange(1 << 23, 1 << 24, dtype=np.int64)
    exact = 3 * m                                  # 1.5 * S in units of 2^-24 (S = m * 2^-23)
    f = (exact.astype(np.float64)).astype(np.float32)
    bits = f.view(np.uint32)
    hit = ((bits & 0xFFFF) == 0x8000) & (f.astype(np.float64) != exact.astype(np.float64))
    ms = m[hit][:count]
    return (ms.astype(np.float64) * 2.0 ** -23).astype(np.float32)


def test_dequantize_single_rounding_at_fp32_ties(oracle):
    s = fp32_tie_scales(256)
    double_rounded = oracle.f32_to_bf16((1.5 * s.astype(np.float64)).astype(np.float32))
    keep = [r for r in range(len(s)) if int(double_rounded[r]) != nearest_bf16_fraction(1.5 * float(s[r]))]
    s = s[keep][:64]
    assert len(s) >= 16
    rows = len(s)
    q = np.full((rows, 8), 0x33, np.uint8)           # every element code 3: e2m1 = 1.5
    q[:, 1] = 0xBB                                   # and -1.5
    sb = np.full((rows, 1), 0x38, np.uint8)          # block scale 1.0
    out = oracle.dequantize_bf16(q, sb, s)
    double_rounded = oracle.f32_to_bf16((1.5 * s.astype(np.float64)).astype(np.float32))
    differs = 0
    for r in range(rows):
        want = nearest_bf16_fraction(1.5 * float(s[r]))
        assert int(out[r, 0]) == want
        assert int(out[r, 2]) == want | 0x8000 or int(out[r, 3]) == want | 0x8000
        differs += int(double_rounded[r]) != want
    assert differs == rows                           # every case separates the two roundings
