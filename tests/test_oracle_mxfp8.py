"""Pins for the oracle's MXFP8 quantizer and GEMM (Miles page, section
MXFP8格式背景: 32 consecutive E4M3 values share one E8M0 power-of-two scale,
rounded up so the block maximum is not clipped).

  - closed form: the scale 2^e is the smallest power of two with
    a_b / 2^e <= 448, checked in exact rational arithmetic; zero blocks
    take code 0;
  - library routine: element codes equal torch's float8_e4m3fn conversion of
    x / 2^e (round to nearest even; sign kept on zeros);
  - round trip: values already on the MXFP8 grid come back unchanged;
  - GEMM: against numpy's matmul of the dequantized operands and an exact
    Fraction dot product on a tiny case.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthgen as sg


def _f32(bf16):
    return (bf16.astype(np.uint32) << 16).view(np.float32)


def test_scale_is_smallest_unclipped_power_of_two(oracle):
    x = sg.student_t3_bf16(3, sg.S_X, (64, 1024))
    x[0, :32] = 0                                   # zero block
    x[1, :32] = 0x7F7F                              # bf16 max
    x[2, 32:64] = 0x0001                            # smallest subnormal
    q, sc = oracle.mxfp8_quantize_rows(x)
    a = np.abs(_f32(x).astype(np.float64)).reshape(64, 32, 32).max(axis=2)
    for r in range(64):
        for b in range(32):
            e = int(sc[r, b]) - 127
            amax = Fraction(float(a[r, b]))
            if amax == 0:
                assert sc[r, b] == 0
                continue
            assert amax <= 448 * Fraction(2) ** e
            assert e == -127 or amax > 448 * Fraction(2) ** (e - 1)


def test_elements_match_torch_float8(oracle):
    x = sg.normal_outliers_bf16(5, sg.S_X, (128, 512), 1.0, 0.02, 300.0)
    x[3, 5] = 0x8000                                # -0
    x[4, 40:64] = 0x8001                            # negative subnormals
    q, sc = oracle.mxfp8_quantize_rows(x)
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    v = torch.from_numpy((_f32(x).astype(np.float64) / scale).astype(np.float32))
    want = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_grid_values_round_trip(oracle):
    e4 = oracle.e4m3_table()
    rng = np.random.default_rng(9)
    rows = []
    for e in range(-20, 21, 4):
        codes = rng.integers(0, 0x7F, 32)
        codes[0] = 0x7E                             # 448: the block max sits at the top
        vals = e4[codes] * 2.0 ** e * rng.choice([-1, 1], 32)
        rows.append(vals)
    x = sg.f32_to_bf16(np.array(rows, np.float32))
    back = _f32(x).astype(np.float64)
    assert np.array_equal(back, np.array(rows))      # the grid values are bf16-exact
    q, sc = oracle.mxfp8_quantize_rows(x)
    assert np.array_equal(oracle.mxfp8_dequantize(q, sc), np.array(rows))


def test_gemm_against_numpy_and_fractions(oracle):
    xa = sg.student_t3_bf16(6, sg.S_X, (37, 256))
    xb = sg.normal_bf16(7, sg.S_W, (29, 256), 0.0, 0.02)
    a = oracle.mxfp8_quantize_rows(xa)
    b = oracle.mxfp8_quantize_rows(xb)
    y, bound = oracle.mxfp8_gemm(a, b)
    da, db = oracle.mxfp8_dequantize(*a), oracle.mxfp8_dequantize(*b)
    assert np.all(np.abs(y - da @ db.T) <= 1e-12 * (np.abs(da) @ np.abs(db).T))
    assert np.allclose(bound, np.abs(da) @ np.abs(db).T, rtol=1e-14)
    # exact on one entry
    exact = sum(Fraction(float(u)) * Fraction(float(v)) for u, v in zip(da[3], db[5]))
    assert Fraction(float(y[3, 5])) == exact or abs(float(exact) - y[3, 5]) <= 1e-15 * bound[3, 5]


def test_rejects_bad_shapes_and_non_finite(oracle):
    with pytest.raises(ValueError):
        oracle.mxfp8_quantize_rows(np.zeros((2, 48), np.uint16))
    x = np.zeros((2, 64), np.uint16)
    x[1, 7] = 0x7F80
    with pytest.raises(ValueError):
        oracle.mxfp8_quantize_rows(x)
