// mxfp8_codec.h -- the MXFP8 element and scale encoders (gfx950) shared by
// the quantizer and the codec self-test library: E8M0 scale code from the
// bf16 bits of a block amax, E4M3 codes by the pack-convert (nearest even,
// sign kept).  The scale rule follows the Miles page, section MXFP8格式背景.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

typedef short s16x2 __attribute__((ext_vector_type(2)));

// E8M0 scale code for a block whose largest magnitude has bf16 bits `a`
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t a) {
  const int ef = (int)(a >> 7);  // biased exponent field (sign already cleared)
  if (ef == 0) return 0u;        // zero or subnormal amax: smallest scale
  const int code = ef - 8 + ((a & 0x7Fu) > 96u ? 1 : 0);
  return (uint32_t)(code < 0 ? 0 : (code > 254 ? 254 : code));
}

// two fp32 values -> two E4M3 codes in the low (SEL = 0) or high 16 bits
template <bool HI>
__device__ __forceinline__ uint32_t fp8_encode2(uint32_t old, float a, float b) {
  s16x2 o = __builtin_bit_cast(s16x2, old);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, 1.0f, HI));
}

__device__ __forceinline__ uint32_t fp8_encode4(uint32_t w0, uint32_t w1, float inv) {
  uint32_t r = fp8_encode2<false>(0u, __uint_as_float(w0 << 16) * inv,
                                  __uint_as_float(w0 & 0xFFFF0000u) * inv);
  return fp8_encode2<true>(r, __uint_as_float(w1 << 16) * inv,
                           __uint_as_float(w1 & 0xFFFF0000u) * inv);
}

}  // namespace nvfp4
