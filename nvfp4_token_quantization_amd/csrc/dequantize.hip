// dequantize.hip -- NVFP4 -> bf16 for backward GEMMs that consume the
// dequantized forward operands (gfx950).
//
// The Miles page (section 反量化反向模式) describes the dequantized-backward
// mode: the backward GEMMs run in BF16 on the BF16 dequantization of the exact
// low-precision forward operands, at the cost of an extra dequantize step.
// Each output is bf16(S * s_b * e2m1(q)) with the product formed exactly and
// rounded once (nearest even): S * s_b is exact in fp64 (24 + 4 significant
// bits) and so is its product with an E2M1 value.  Rounding that double to
// fp32 and then to bf16 is a single rounding except when the fp32 value is
// exactly a bf16 halfway point while the double is not; there the direction
// comes from comparing the double with the fp32 value.
//
// One thread per 16-element block: 8 bytes of codes and one scale byte in,
// 32 bytes of bf16 out; consecutive threads take consecutive blocks, so the
// whole [rows, k] tensor is one flat, fully coalesced stream.
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_of_exact(double x) {
  const float f = (float)x;
  const uint32_t u = __float_as_uint(f);
  uint32_t b = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  if (__builtin_expect((u & 0xFFFFu) == 0x8000u, 0)) {
    const double fd = (double)f;
    if (fd != x) b = (__builtin_fabs(x) > __builtin_fabs(fd)) ? (u >> 16) + 1u : (u >> 16);
  }
  return b;
}

template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t codes, double sd) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
  return bf16_of_exact(sd * (double)v.x) | (bf16_of_exact(sd * (double)v.y) << 16);
}

template <typename IDX>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ sb,
                                                         const float* __restrict__ s,
                                                         IDX nblocks, IDX blocks_per_scale,
                                                         uint16_t* __restrict__ out) {
  const IDX stride = (IDX)gridDim.x * 256;
  for (IDX b = (IDX)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += stride) {
    const uint2 c = reinterpret_cast<const uint2*>(q)[b];
    const double sd = (double)s[b / blocks_per_scale] * (double)e4m3_decode(sb[b] & 0x7Fu);
    uint4 lo, hi;
    lo.x = dequant_pair<0>(c.x, sd);
    lo.y = dequant_pair<1>(c.x, sd);
    lo.z = dequant_pair<2>(c.x, sd);
    lo.w = dequant_pair<3>(c.x, sd);
    hi.x = dequant_pair<0>(c.y, sd);
    hi.y = dequant_pair<1>(c.y, sd);
    hi.z = dequant_pair<2>(c.y, sd);
    hi.w = dequant_pair<3>(c.y, sd);
    uint4* o = reinterpret_cast<uint4*>(out) + 2 * (int64_t)b;
    o[0] = lo;
    o[1] = hi;
  }
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_dequantize_rows(const uint8_t* q, const uint8_t* sb, const float* s,
                                     int64_t rows, int64_t k, int64_t rows_per_scale,
                                     uint16_t* x_bf16, void* stream) {
  if (rows < 0 || k < 0 || rows_per_scale < 1) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 16 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (rows == 0 || k == 0) return NVFP4_SUCCESS;
  if (!q || !sb || !s || !x_bf16) return NVFP4_ERROR_INVALID_VALUE;
  if (rows > ((int64_t)1 << 36) || k > ((int64_t)1 << 30)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(q, 16) || !aligned(s, 4) || !aligned(x_bf16, 16)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  const int64_t nblocks = rows * (k / 16);
  const int64_t bps = rows_per_scale * (k / 16);
  const int64_t need = (nblocks + 255) / 256;
  const int64_t cap = (int64_t)nvfp4host::num_cus() * 16;
  dim3 grid((unsigned)(need < cap ? need : cap));
  hipStream_t str = (hipStream_t)stream;
  if (nblocks < ((int64_t)1 << 31))
    hipLaunchKernelGGL(nvfp4::dequantize_kernel<uint32_t>, grid, dim3(256), 0, str, q, sb, s,
                       (uint32_t)nblocks, (uint32_t)(bps < nblocks ? bps : nblocks), x_bf16);
  else
    hipLaunchKernelGGL(nvfp4::dequantize_kernel<uint64_t>, grid, dim3(256), 0, str, q, sb, s,
                       (uint64_t)nblocks, (uint64_t)bps, x_bf16);
  return nvfp4host::launch_status();
}
