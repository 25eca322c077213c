// mxfp8.hip -- MXFP8 quantization (gfx950): 32 consecutive values along K
// share one E8M0 power-of-two scale, values are E4M3.
//
// The Miles page (section MXFP8格式背景) describes the format and its scale
// rule: the decoded scale is rounded up so the block maximum is never
// clipped.  Here 2^e is the smallest power of two with a_b / 2^e <= 448,
// computed exactly from the bf16 bits of the block amax a_b = m 2^E
// (1 <= m < 2): e = E - 8 when m <= 1.75 (448 = 1.75 * 2^8), else E - 7.
// Code e + 127 is clamped to [0, 254]; zero and subnormal-amax blocks take 0.
// Elements: x * 2^-e is exact (a power-of-two scaling; results below 2^-126
// are far under E4M3's smallest step and round to zero either way) and
// gfx950's pack-convert rounds it to E4M3 (nearest even, sign kept).
//
// One thread per 32-element block over the flat [rows, k] tensor: 64 bytes
// in, 32 + 1 bytes out, consecutive threads on consecutive blocks.
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

template <typename IDX>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t* __restrict__ x,
                                                             IDX nblocks, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sc) {
  const IDX stride = (IDX)gridDim.x * 256;
  for (IDX b = (IDX)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += stride) {
    const uint4* xb = reinterpret_cast<const uint4*>(x) + 4 * (int64_t)b;
    const uint4 v0 = ld_stream(xb), v1 = ld_stream(xb + 1), v2 = ld_stream(xb + 2),
                v3 = ld_stream(xb + 3);
    const uint32_t a = max(block_amax_bits(v0, v1), block_amax_bits(v2, v3));
    const uint32_t code = mx_scale_code(a);
    const float inv = __uint_as_float((254u - code) << 23);  // 2^-(code - 127)
    uint4 o0, o1;
    o0.x = fp8_encode4(v0.x, v0.y, inv);
    o0.y = fp8_encode4(v0.z, v0.w, inv);
    o0.z = fp8_encode4(v1.x, v1.y, inv);
    o0.w = fp8_encode4(v1.z, v1.w, inv);
    o1.x = fp8_encode4(v2.x, v2.y, inv);
    o1.y = fp8_encode4(v2.z, v2.w, inv);
    o1.z = fp8_encode4(v3.x, v3.y, inv);
    o1.w = fp8_encode4(v3.z, v3.w, inv);
    uint4* qo = reinterpret_cast<uint4*>(q) + 2 * (int64_t)b;
    qo[0] = o0;
    qo[1] = o1;
    sc[b] = (uint8_t)code;
  }
}

__global__ __launch_bounds__(256) void debug_fp8_kernel(const float* __restrict__ v, int64_t n,
                                                        uint8_t* __restrict__ code) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    code[i] = (uint8_t)(fp8_encode2<false>(0u, v[i], 0.0f) & 0xFFu);
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_mxfp8_quantize_rows(const uint16_t* x_bf16, int64_t rows, int64_t k,
                                         uint8_t* q, uint8_t* sc, void* stream) {
  if (rows < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 32 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (rows == 0 || k == 0) return NVFP4_SUCCESS;
  if (!x_bf16 || !q || !sc) return NVFP4_ERROR_INVALID_VALUE;
  if (rows > ((int64_t)1 << 36) || k > ((int64_t)1 << 30)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  const int64_t nblocks = rows * (k / 32);
  const int64_t need = (nblocks + 255) / 256;
  const int64_t cap = (int64_t)nvfp4host::num_cus() * 16;
  dim3 grid((unsigned)(need < cap ? need : cap));
  hipStream_t str = (hipStream_t)stream;
  if (nblocks < ((int64_t)1 << 31))
    hipLaunchKernelGGL(nvfp4::mxfp8_quantize_kernel<uint32_t>, grid, dim3(256), 0, str, x_bf16,
                       (uint32_t)nblocks, q, sc);
  else
    hipLaunchKernelGGL(nvfp4::mxfp8_quantize_kernel<uint64_t>, grid, dim3(256), 0, str, x_bf16,
                       (uint64_t)nblocks, q, sc);
  return nvfp4host::launch_status();
}

extern "C" int nvfp4_debug_encode_fp8(const float* v, int64_t n, uint8_t* code, void* stream) {
  if (n < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (n == 0) return NVFP4_SUCCESS;
  if (!v || !code) return NVFP4_ERROR_INVALID_VALUE;
  if (!aligned(v, 4)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  const int64_t need = (n + 255) / 256;
  dim3 grid((unsigned)(need < 4096 ? need : 4096));
  hipLaunchKernelGGL(nvfp4::debug_fp8_kernel, grid, dim3(256), 0, (hipStream_t)stream, v, n, code);
  return nvfp4host::launch_status();
}
