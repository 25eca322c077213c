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
// Layout: L lanes of a wave64 own a row (L = 16, 32 or 64) and lane j owns
// the row's 8-element half-blocks j, j+L, ..., so every store instruction
// writes L * 16 contiguous bytes of bf16 and every code load reads L * 4
// contiguous bytes; rows longer than L * U half-blocks are walked in chunks.
//
// Arithmetic: w = s_b * e2m1 is exact in fp32 (at most 6 significant bits,
// never below 2^-10), so S * w needs one rounding: t = fl32(S * w), and
// v_cvt_pk_bf16_f32 rounds t to the nearest bf16.  That equals the single
// rounding of the exact product unless t is itself a bf16 halfway point
// (low 16 bits 0x8000) while the product is not, or t is below 2^-100
// (where the residual of the product need not be representable).  A wave
// with such an element in a half-block redoes the half-block in fp64 (exact
// product, direction fixed by comparing the double with its fp32 rounding).
#include "nvfp4_internal.h"

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ uint32_t dequant_pair_exact(uint32_t codes, double sd) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
  return bf16_of_exact(sd * (double)v.x) | (bf16_of_exact(sd * (double)v.y) << 16);
}

// True when fl32 value t is a bf16 halfway point, or nonzero and below
// 2^-100.  Zeros are exact products (with the sign of the E2M1 code).
__device__ __forceinline__ bool needs_exact(float t) {
  const uint32_t u = __float_as_uint(t);
  return (u & 0xFFFFu) == 0x8000u || (u & 0x7FFFFFFFu) - 1u < (27u << 23) - 1u;
}

template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair_fast(uint32_t codes, float S, float sbv,
                                                      bool& slow) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
  const float t0 = S * (v.x * sbv), t1 = S * (v.y * sbv);
  slow = slow || needs_exact(t0) || needs_exact(t1);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){t0, t1}, bf16x2));
}

__device__ __forceinline__ uint4 dequant_half(uint32_t codes, float S, uint32_t sb_code) {
  const float sbv = e4m3_decode(sb_code & 0x7Fu);
  bool slow = false;
  uint4 o;
  o.x = dequant_pair_fast<0>(codes, S, sbv, slow);
  o.y = dequant_pair_fast<1>(codes, S, sbv, slow);
  o.z = dequant_pair_fast<2>(codes, S, sbv, slow);
  o.w = dequant_pair_fast<3>(codes, S, sbv, slow);
  if (__builtin_expect(slow, 0)) {
    const double sd = (double)S * (double)sbv;
    o.x = dequant_pair_exact<0>(codes, sd);
    o.y = dequant_pair_exact<1>(codes, sd);
    o.z = dequant_pair_exact<2>(codes, sd);
    o.w = dequant_pair_exact<3>(codes, sd);
  }
  return o;
}

// One row per L lanes, U half-blocks per lane per chunk; a wave takes 64 / L
// rows per row group and walks row groups with a grid stride (wave-uniform).
template <int L, int U>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t* __restrict__ q,
                                                         const uint8_t* __restrict__ sb,
                                                         const float* __restrict__ s,
                                                         int64_t rows, int nh,
                                                         int64_t rows_per_scale,
                                                         uint16_t* __restrict__ out) {
  constexpr int RPW = 64 / L;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int sub = lane / L;
  const int64_t ngroups = (rows + RPW - 1) / RPW;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); g < ngroups; g += stride) {
    const int64_t row = g * RPW + sub;
    const bool row_ok = row < rows;
    const float S = row_ok ? s[row / rows_per_scale] : 0.0f;
    const uint32_t* qr = q + (row_ok ? row : 0) * nh;
    const uint8_t* sr = sb + (row_ok ? row : 0) * (nh / 2);
    uint4* orow = reinterpret_cast<uint4*>(out + (row_ok ? row : 0) * (int64_t)nh * 8);
    for (int h0 = 0; h0 < nh; h0 += L * U) {
      uint32_t c[U], b[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int h = h0 + j + L * i;
        const bool ok = row_ok && h < nh;
        c[i] = ok ? qr[h] : 0u;
        b[i] = ok ? sr[h >> 1] : 0u;
      }
      // streaming stores: the output is four times the input and is not
      // read again here (cached stores run this write-heavy stream at about
      // 60% of the rate)
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int h = h0 + j + L * i;
        if (row_ok && h < nh)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, dequant_half(c[i], S, b[i])),
                                      reinterpret_cast<u32x4*>(orow) + h);
      }
    }
  }
}

typedef void (*DeqKernel)(const uint32_t*, const uint8_t*, const float*, int64_t, int, int64_t,
                          uint16_t*);

// The widest lane group whose chunk covers the row's half-blocks evenly,
// else 64 lanes with 8 half-blocks per lane per chunk.
static DeqKernel pick_dequant_kernel(int nh, int& lanes) {
#define NVFP4_DQ(L)                                                  \
  switch (nh / L) {                                                  \
    case 1: lanes = L; return dequantize_kernel<L, 1>;               \
    case 2: lanes = L; return dequantize_kernel<L, 2>;               \
    case 3: lanes = L; return dequantize_kernel<L, 3>;               \
    case 4: lanes = L; return dequantize_kernel<L, 4>;               \
    case 5: lanes = L; return dequantize_kernel<L, 5>;               \
    case 6: lanes = L; return dequantize_kernel<L, 6>;               \
    case 8: lanes = L; return dequantize_kernel<L, 8>;               \
    default: break;                                                  \
  }
  if (nh % 64 == 0) { NVFP4_DQ(64) }
  if (nh % 32 == 0) { NVFP4_DQ(32) }
  if (nh % 16 == 0) { NVFP4_DQ(16) }
#undef NVFP4_DQ
  if (nh <= 16) { lanes = 16; return dequantize_kernel<16, 1>; }
  if (nh <= 32) { lanes = 32; return dequantize_kernel<32, 1>; }
  lanes = 64;
  return dequantize_kernel<64, 8>;
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
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.e4m3_codes(sb, rows * (k / 16));
    chk.f32_finite(s, (rows + rows_per_scale - 1) / rows_per_scale);
    if ((st = chk.result())) return st;
  }
#endif
  const int nh = (int)(k / 8);  // 8-element half-blocks per row
  int lanes = 64;
  nvfp4::DeqKernel kern = nvfp4::pick_dequant_kernel(nh, lanes);
  const int64_t row_groups = (rows + 64 / lanes - 1) / (64 / lanes);
  const int64_t need = (row_groups + 3) / 4;
  const int64_t cap = (int64_t)nvfp4host::num_cus() * 32;
  dim3 grid((unsigned)(need < cap ? need : cap));
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint32_t*>(q), sb, s, rows, nh, rows_per_scale, x_bf16);
  return nvfp4host::launch_status();
}
