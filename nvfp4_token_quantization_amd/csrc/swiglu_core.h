// swiglu_core.h -- the SwiGLU element arithmetic shared by the fused SwiGLU
// -> requantize kernel and the grouped GEMM's SwiGLU epilogue (gfx950):
// h = bf16(fl32(g * u / (1 + exp(-g)))), the quotient formed in fp64 (g * u
// is exact there) or, for all but about 1 element in 2000, by an fp32
// evaluation with a rounding test that returns the same bf16.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

// fp32 -> bf16 bit pattern, round to nearest even (finite input; values at or
// past the halfway point above the largest bf16 become infinity, as in IEEE).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Reference evaluation: the quotient in fp64 (g * u is exact there).
__device__ __forceinline__ uint32_t swiglu_bf16_fp64(float g, float u) {
  const double gd = g, ud = u;
  const double h = (gd * ud) / (1.0 + exp(-gd));
  return bf16_rne((float)h);
}

// Fast evaluation with a rounding test (Ziv's strategy).  exp(-g) comes from
// a Cody-Waite reduction by ln 2 and a degree-7 Taylor polynomial, and
// 1 / (1 + exp(-g)) from a hardware reciprocal (1 ulp) refined by one Newton
// step; over every fp32 g in [-80, 100] this factor is within 2.6 units of
// 2^-24 relative of the exact sigmoid (an exhaustive sweep with the
// reciprocal's result taken exact, one ulp high and one ulp low).  Two more
// roundings (g * u, and the product) bring h_f within 3.6 units, so
// fl32(h_exact) lies within 5 fp32 ulps of h_f.  Unless h_f's low 16 bits
// are within 16 ulps of a bf16 halfway point (0x8000), both round to the
// same bf16, and that is the result; otherwise (about 1 element in 2000),
// and for g < -80, results below 2^-100 or at least 2^127, zeros and
// non-finite values, the fp64 evaluation decides.
__device__ __forceinline__ uint32_t swiglu_bf16(float g, float u) {
  const float x = -g;
  float e = 0.0f;
  if (g < 20.0f) {  // for g >= 20, exp(-g) < 2^-28 and 1 + e rounds to 1
    const float n = __builtin_rintf(x * 1.44269504f);
    float r = __builtin_fmaf(-n, 0.693145751953125f, x);  // ln 2, high part (exact product)
    r = __builtin_fmaf(-n, 1.42860677e-06f, r);           // ln 2, low part
    float p = __builtin_fmaf(r, 1.98412701e-04f, 1.38888892e-03f);
    p = __builtin_fmaf(p, r, 8.33333377e-03f);
    p = __builtin_fmaf(p, r, 4.16666679e-02f);
    p = __builtin_fmaf(p, r, 1.66666672e-01f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    e = __builtin_ldexpf(p, (int)n);
  }
  const float d = 1.0f + e;
  float rc = __builtin_amdgcn_rcpf(d);
  rc = __builtin_fmaf(__builtin_fmaf(-d, rc, 1.0f), rc, rc);
  const float h = (g * u) * rc;
  const uint32_t b = __float_as_uint(h);
  const uint32_t lo = b & 0xFFFFu;
  const bool unsafe = (lo >= 0x8000u - 16u && lo <= 0x8000u + 16u) || !(g >= -80.0f) ||
                      !(__builtin_fabsf(h) >= 0x1p-100f) || !(__builtin_fabsf(h) < 0x1p127f);
  if (__builtin_expect(unsafe, 0)) return swiglu_bf16_fp64(g, u);
  return bf16_rne(h);
}

}  // namespace nvfp4
