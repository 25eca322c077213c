"""Pins for the oracle's bf16 rounding and SwiGLU (CPU only).

The SwiGLU -> per-token requantize chain is the fused form of the pages'
"amax reuse" and "fusion" (miniTE page, section Transformer Engine路径优化);
the gate and up projections come from one fused GEMM (Miles page, section
并行度与张量转换的一致性契约).  Pins:
  - fp32 -> bf16 rounding against torch's conversion (a library routine) on
    every exponent with the tie / near-tie / overflow mantissa patterns, and on
    random bit patterns;
  - SwiGLU against torch's fp64 silu times up, rounded by torch, over several
    magnitude ranges (a dropped term, swapped halves or a sign slip in the
    exponent fails these);
  - closed forms: for g >= 40 the sigmoid is 1 to fp64 precision, so
    h = bf16(fl32(g * u)); zeros keep the sign of g * u; very negative g
    underflows to a signed zero;
  - the chain: quantizing H with its own row amax passed in equals quantizing
    it from scratch (amax reuse leaves the bits unchanged).
"""
import numpy as np
import pytest
import torch


def _torch_bf16_bits(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().astype(np.uint16)


def _patterns():
    hi7 = np.array([0, 1, 0x3F, 0x40, 0x7E, 0x7F], np.uint32)
    lo16 = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234], np.uint32)
    exps = np.arange(0, 255, dtype=np.uint32)
    e, h, l, s = np.meshgrid(exps, hi7, lo16, np.array([0, 1], np.uint32), indexing="ij")
    bits = (s << 31) | (e << 23) | (h << 16) | l
    return bits.reshape(-1).view(np.float32)


def test_bf16_rounding_structured(oracle):
    v = _patterns()
    assert np.array_equal(oracle.f32_to_bf16(v), _torch_bf16_bits(v))


def test_bf16_rounding_random_bits(oracle):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.f32_to_bf16(v), _torch_bf16_bits(v))


def test_bf16_rounding_overflow_and_ties(oracle):
    cases = {
        0x7F7F7FFF: 0x7F7F,  # below the halfway point to 2^128: stays finite
        0x7F7F8000: 0x7F80,  # halfway: ties to the even pattern, which is inf
        0x3F808000: 0x3F80,  # tie between 0x3F80 and 0x3F81: even wins
        0x3F818000: 0x3F82,  # tie between 0x3F81 and 0x3F82: even wins
        0x00008000: 0x0000,  # tie at the bottom of the subnormals
        0x00018000: 0x0002,
        0x80018001: 0x8002,  # negative, just above the tie
    }
    v = np.array(list(cases), np.uint32).view(np.float32)
    assert [int(x) for x in oracle.f32_to_bf16(v)] == list(cases.values())


def _torch_swiglu(g, u):
    g64 = torch.from_numpy(g.astype(np.float64))
    u64 = torch.from_numpy(u.astype(np.float64))
    h = torch.nn.functional.silu(g64) * u64
    return h.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


@pytest.mark.parametrize("gstd,ustd", [(0.5, 1.0), (3.0, 0.02), (30.0, 5.0), (1e-3, 1e3)])
def test_swiglu_against_torch_fp64(oracle, gstd, ustd):
    rng = np.random.default_rng(int(gstd * 1000) + 3)
    rows, f = 64, 1024
    g = (rng.standard_normal((rows, f)) * gstd).astype(np.float32)
    u = (rng.standard_normal((rows, f)) * ustd).astype(np.float32)
    h = oracle.swiglu_rows(np.concatenate([g, u], axis=1))
    assert np.array_equal(h, _torch_swiglu(g, u))
    # the halves are not interchangeable
    h_swapped = oracle.swiglu_rows(np.concatenate([u, g], axis=1))
    assert not np.array_equal(h_swapped, h)


def test_swiglu_log_uniform_magnitudes(oracle):
    rng = np.random.default_rng(11)
    n = 1 << 18
    g = (np.exp(rng.uniform(-20, 5, n)) * rng.choice([-1, 1], n)).astype(np.float32)
    u = (np.exp(rng.uniform(-20, 20, n)) * rng.choice([-1, 1], n)).astype(np.float32)
    h = oracle.swiglu_rows(np.stack([g, u], axis=0).reshape(1, 2 * n))
    assert np.array_equal(h.reshape(-1), _torch_swiglu(g, u))


def test_swiglu_closed_forms(oracle):
    g = np.array([40.0, 55.5, 1000.0, 0.0, -0.0, 0.0, -2000.0, -2000.0, 3.0], np.float32)
    u = np.array([1.7, -3.25, 1e-3, -1.0, -1.0, 0.0, 1.0, -1.0, 0.0], np.float32)
    h = oracle.swiglu_rows(np.concatenate([g, u])[None, :])[0]
    # sigmoid(g) == 1 in fp64 for g >= 40: h = bf16(fl32(g * u))
    assert np.array_equal(h[:3], oracle.f32_to_bf16((g[:3].astype(np.float64) * u[:3]).astype(np.float32)))
    # signed zeros: sign of g * u
    assert [int(x) for x in h[3:]] == [0x8000, 0x0000, 0x0000, 0x8000, 0x0000, 0x0000]


def test_swiglu_rejects_non_finite(oracle):
    gu = np.ones((2, 32), np.float32)
    gu[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.swiglu_rows(gu)
    big = np.full((1, 32), 3e38, np.float32)  # g * u overflows fp32
    with pytest.raises(ValueError):
        oracle.swiglu_rows(big)


def test_swiglu_empty(oracle):
    assert oracle.swiglu_rows(np.zeros((0, 64), np.float32)).shape == (0, 32)
    assert oracle.swiglu_rows(np.zeros((3, 0), np.float32)).shape == (3, 0)


def test_swiglu_quantize_chain_is_amax_reuse(oracle):
    rng = np.random.default_rng(5)
    gu = (rng.standard_normal((48, 2 * 768)) * 2.0).astype(np.float32)
    h, amax, q, sb, s = oracle.swiglu_quantize_rows(gu)
    hf = (h.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(amax, np.abs(hf).max(axis=1))
    q2, sb2, s2 = oracle.quantize_rows(h, amax_in=amax)
    assert np.array_equal(q, q2) and np.array_equal(sb, sb2)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
