// quantize.hip -- per-token and per-tensor / per-expert NVFP4 quantization
// for gfx950.
//
// Method: the Miles page ("Towards Blackwell-Native 8-bit and 4-bit RL"),
// section 速读 (X ~ s_token * s_block * X_FP4, 16 E2M1 values per E4M3 block
// scale) and section 单Token缩放的在线计算实现 (the FP32 per-token scale is
// computed online in the same call that emits the packed FP4 values and the
// E4M3 scales); the TRIAGE page, section 前置知识, for the decode
// x_hat = S * s_b * Q_E2M1(x / (S * s_b)).
//
// Kernel layout (HBM-bound: 2.5625 bytes move per element):
//  - L lanes of a wave64 own one row (L = 16, 32 or 64 chosen so the row's
//    16-element blocks divide evenly); lane j owns blocks j, j+L, j+2L, ...
//    and keeps them in VGPRs, so the row is read from HBM once.
//  - Each block is 32 contiguous bytes (two 16-byte loads); consecutive
//    lanes read consecutive blocks, so a wave's loads are contiguous.
//  - Block amax: packed 16-bit max over the bf16 magnitude bits (exact:
//    non-negative bf16 bit patterns order like their values).
//  - Row amax: DPP / ds_swizzle / readlane max over the row's lanes.
//  - Per block one correctly rounded division (a_b / 6S) and one correctly
//    rounded reciprocal (1 / d); per element one fp32 multiply and half of a
//    gfx950 pack-convert to E2M1 (two elements per instruction).
#include "nvfp4_internal.h"

namespace nvfp4 {

enum QuantMode { MODE_ROW = 0, MODE_AMAX_IN = 1, MODE_GROUP = 2 };

#ifndef NVFP4_Q_WAVES_PER_SIMD
#define NVFP4_Q_WAVES_PER_SIMD 8
#endif

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Encode one block of 16 elements (two uint4 of bf16) with reciprocal `inv`
// into 8 bytes of E2M1 codes.  When inv is +inf (d is a tiny denormal) x * inv
// would be NaN for x = +-0, so zeros are passed through unchanged there.
__device__ __forceinline__ uint2 encode_block(const uint4& a, const uint4& b, float inv) {
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float r[16];
  if (__builtin_expect(__builtin_isinf(inv), 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float lo = bf16lo(w[i]), hi = bf16hi(w[i]);
      r[2 * i] = (lo == 0.0f) ? lo : lo * inv;
      r[2 * i + 1] = (hi == 0.0f) ? hi : hi * inv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r[2 * i] = bf16lo(w[i]) * inv;
      r[2 * i + 1] = bf16hi(w[i]) * inv;
    }
  }
  uint32_t q0 = 0, q1 = 0;
  q0 = e2m1_encode2<0>(q0, r[0], r[1]);
  q0 = e2m1_encode2<1>(q0, r[2], r[3]);
  q0 = e2m1_encode2<2>(q0, r[4], r[5]);
  q0 = e2m1_encode2<3>(q0, r[6], r[7]);
  q1 = e2m1_encode2<0>(q1, r[8], r[9]);
  q1 = e2m1_encode2<1>(q1, r[10], r[11]);
  q1 = e2m1_encode2<2>(q1, r[12], r[13]);
  q1 = e2m1_encode2<3>(q1, r[14], r[15]);
  return make_uint2(q0, q1);
}

// The NB blocks of one row group held by a lane (one 32-byte block is two
// uint4 of bf16).
template <int NB>
struct RowData {
  uint4 d[NB][2];
};

template <int L, int NB>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t k,
                                          int nblk, int64_t row, int j, RowData<NB>& r) {
  const bool row_ok = row < rows;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (row_ok ? row : 0) * k);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = j + L * i;
    if (row_ok && b < nblk) {
      r.d[i][0] = ld_stream(xr + 2 * b);
      r.d[i][1] = ld_stream(xr + 2 * b + 1);
    } else {
      r.d[i][0] = make_uint4(0, 0, 0, 0);
      r.d[i][1] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Encode and store one row group.  Must be called by all 64 lanes of the
// wave (the row amax is a cross-lane reduction).
template <int L, int NB, int MODE>
__device__ __forceinline__ void encode_rows(const RowData<NB>& r, int64_t rows, int64_t k,
                                            int nblk, int64_t row, int j,
                                            const float* __restrict__ amax_src,
                                            int64_t rows_per_group, uint8_t* __restrict__ q,
                                            uint8_t* __restrict__ sb, float* __restrict__ s) {
  const bool row_ok = row < rows;
  uint32_t bmax[NB];
  uint32_t rmax = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    bmax[i] = block_amax_bits(r.d[i][0], r.d[i][1]);
    rmax = max(rmax, bmax[i]);
  }
  float amax;
  if (MODE == MODE_ROW) {
    amax = __uint_as_float(group_max_u32<L>(rmax) << 16);
  } else if (MODE == MODE_AMAX_IN) {
    amax = row_ok ? amax_src[row] : 0.0f;
  } else {
    amax = row_ok ? amax_src[row / rows_per_group] : 0.0f;
  }
  const float S = amax / 2688.0f;
  if (MODE != MODE_GROUP && row_ok && j == 0) s[row] = S;
  const float t = 6.0f * S;
  uint8_t* qr = q + (row_ok ? row : 0) * (k / 2);
  uint8_t* sr = sb + (row_ok ? row : 0) * (k / 16);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = j + L * i;
    if (row_ok && b < nblk) {
      uint32_t code;
      float inv;
      block_scale(bmax[i], S, t, code, inv);
      reinterpret_cast<uint2*>(qr)[b] = encode_block(r.d[i][0], r.d[i][1], inv);
      sr[b] = (uint8_t)code;
    }
  }
}

// One row per L lanes (NB blocks per lane at most, nblk <= L * NB); a wave
// handles 64 / L rows per row group and walks row groups with a grid stride,
// loading group i + 1 while it encodes group i (two register buffers,
// unrolled by two so the buffers never move).
template <int L, int NB, int MODE>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int nblk,
    const float* __restrict__ amax_src, int64_t rows_per_group, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sb, float* __restrict__ s) {
  constexpr int RPW = 64 / L;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int sub = lane / L;
  const int64_t ngroups = (rows + RPW - 1) / RPW;
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t g0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // wave-uniform
  RowData<NB> r0, r1;
  if (g0 < ngroups) load_rows<L, NB>(x, rows, k, nblk, g0 * RPW + sub, j, r0);
  for (; g0 < ngroups; g0 += 2 * stride) {
    const int64_t g1 = g0 + stride, g2 = g1 + stride;
    if (g1 < ngroups) load_rows<L, NB>(x, rows, k, nblk, g1 * RPW + sub, j, r1);
    encode_rows<L, NB, MODE>(r0, rows, k, nblk, g0 * RPW + sub, j, amax_src, rows_per_group, q,
                             sb, s);
    if (g2 < ngroups) load_rows<L, NB>(x, rows, k, nblk, g2 * RPW + sub, j, r0);
    if (g1 < ngroups)
      encode_rows<L, NB, MODE>(r1, rows, k, nblk, g1 * RPW + sub, j, amax_src, rows_per_group,
                               q, sb, s);
  }
}

// Rows longer than 64 * 8 blocks: one wave per row, two passes (the second
// re-reads the row, mostly from L2).
template <int MODE>
__global__ __launch_bounds__(256) void quantize_rows_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int nblk,
    const float* __restrict__ amax_src, int64_t rows_per_group, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sb, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * k);
  float amax;
  if (MODE == MODE_ROW) {
    uint32_t rmax = 0;
    for (int b = lane; b < nblk; b += 64) rmax = max(rmax, block_amax_bits(xr[2 * b], xr[2 * b + 1]));
    amax = __uint_as_float(group_max_u32<64>(rmax) << 16);
  } else if (MODE == MODE_AMAX_IN) {
    amax = amax_src[row];
  } else {
    amax = amax_src[row / rows_per_group];
  }
  const float S = amax / 2688.0f;
  if (MODE != MODE_GROUP && lane == 0) s[row] = S;
  const float t = 6.0f * S;
  uint8_t* qr = q + row * (k / 2);
  uint8_t* sr = sb + row * (k / 16);
  for (int b = lane; b < nblk; b += 64) {
    uint4 a0 = xr[2 * b], a1 = xr[2 * b + 1];
    uint32_t code;
    float inv;
    block_scale(block_amax_bits(a0, a1), S, t, code, inv);
    reinterpret_cast<uint2*>(qr)[b] = encode_block(a0, a1, inv);
    sr[b] = (uint8_t)code;
  }
}

// Rows with k == 0: only the outer scale is written (amax of an empty row is 0).
template <int MODE>
__global__ __launch_bounds__(256) void quantize_empty_rows_kernel(int64_t rows,
                                                                  const float* __restrict__ amax_src,
                                                                  float* __restrict__ s) {
  int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < rows) s[r] = (MODE == MODE_AMAX_IN ? amax_src[r] : 0.0f) / 2688.0f;
}

// ---------------------------------------------------------------- weights --
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.0f;
}

// Group amax: block (g, c) reduces chunk c of group g's contiguous elements
// (4 independent 16-byte streaming loads in flight per thread) and folds it
// into amax[g] with an atomic max on the bit pattern (order independent, so
// the result is deterministic).
__global__ __launch_bounds__(256) void group_amax_kernel(const uint16_t* __restrict__ w,
                                                         int64_t group_elems, int64_t chunk_vecs,
                                                         int chunks, float* __restrict__ amax) {
  __shared__ uint32_t red[4];
  const int64_t g = blockIdx.x / chunks;
  const int64_t c = blockIdx.x % chunks;
  const int64_t nvec = group_elems / 8;  // 16-byte vectors in the group
  const uint4* base = reinterpret_cast<const uint4*>(w + g * group_elems);
  const int64_t v0 = c * chunk_vecs;
  const int64_t v1 = min(nvec, v0 + chunk_vecs);
  uint32_t m = 0;
  int64_t v = v0 + threadIdx.x;
  for (; v + 3 * 256 < v1; v += 4 * 256) {
    uint4 a = ld_stream(base + v), b = ld_stream(base + v + 256);
    uint4 c2 = ld_stream(base + v + 512), d = ld_stream(base + v + 768);
    m = max(m, max(block_amax_bits(a, b), block_amax_bits(c2, d)));
  }
  for (; v < v1; v += 256) m = max(m, block_amax_bits(base[v], make_uint4(0, 0, 0, 0)));
  m = group_max_u32<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = max(max(red[0], red[1]), max(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax + g), r << 16);
  }
}

// S[g] = amax[g] / 2688 (and amax_out = amax_in when the amax was supplied).
__global__ __launch_bounds__(256) void group_scale_kernel(int64_t groups,
                                                          const float* __restrict__ amax_in,
                                                          float* __restrict__ amax_out,
                                                          float* __restrict__ s) {
  int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  float a = amax_in ? amax_in[g] : amax_out[g];
  if (amax_in && amax_out) amax_out[g] = a;
  s[g] = a / 2688.0f;
}

// ------------------------------------------------------------ dispatching --
typedef void (*RowKernel)(const uint16_t*, int64_t, int64_t, int, const float*, int64_t, uint8_t*,
                          uint8_t*, float*);

template <int MODE>
static RowKernel pick_row_kernel(int nblk, int& lanes) {
#define NVFP4_PICK(L)                                                            \
  switch ((nblk + L - 1) / L) {                                                  \
    case 1: lanes = L; return quantize_rows_kernel<L, 1, MODE>;                  \
    case 2: lanes = L; return quantize_rows_kernel<L, 2, MODE>;                  \
    case 3: lanes = L; return quantize_rows_kernel<L, 3, MODE>;                  \
    case 4: lanes = L; return quantize_rows_kernel<L, 4, MODE>;                  \
    case 5: lanes = L; return quantize_rows_kernel<L, 5, MODE>;                  \
    case 6: lanes = L; return quantize_rows_kernel<L, 6, MODE>;                  \
    case 7:                                                                      \
    case 8: lanes = L; return quantize_rows_kernel<L, 8, MODE>;                  \
    default: break;                                                              \
  }
  // prefer the widest group that divides the row's blocks evenly
  if (nblk % 64 == 0 && nblk / 64 <= 8) { NVFP4_PICK(64) }
  if (nblk % 32 == 0 && nblk / 32 <= 8) { NVFP4_PICK(32) }
  if (nblk % 16 == 0 && nblk / 16 <= 8) { NVFP4_PICK(16) }
  if (nblk <= 16 * 8 && nblk < 32) { NVFP4_PICK(16) }
  if (nblk <= 32 * 8 && nblk < 64) { NVFP4_PICK(32) }
  if (nblk <= 64 * 8) { NVFP4_PICK(64) }
#undef NVFP4_PICK
  lanes = 0;
  return nullptr;
}

template <int MODE>
static void launch_rows(const uint16_t* x, int64_t rows, int64_t k, const float* amax_src,
                        int64_t rows_per_group, uint8_t* q, uint8_t* sb, float* s,
                        hipStream_t stream) {
  const int nblk = (int)(k / 16);
  int lanes = 0;
  RowKernel kern = pick_row_kernel<MODE>(nblk, lanes);
  if (kern) {
    // enough resident waves to keep HBM busy, and several row groups per wave
    // so loads overlap encoding (NVFP4_Q_WAVES_PER_SIMD waves per SIMD)
    const int64_t rows_per_block = 4 * (64 / lanes);
    const int64_t need = (rows + rows_per_block - 1) / rows_per_block;
    const int64_t cap = (int64_t)nvfp4host::num_cus() * NVFP4_Q_WAVES_PER_SIMD;
    dim3 grid((unsigned)(need < cap ? need : cap));
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, x, rows, k, nblk, amax_src,
                       rows_per_group, q, sb, s);
  } else {
    dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(quantize_rows_long_kernel<MODE>, grid, dim3(256), 0, stream, x, rows, k,
                       nblk, amax_src, rows_per_group, q, sb, s);
  }
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_quantize_rows(const uint16_t* x_bf16, int64_t rows, int64_t k,
                                   const float* amax_in, uint8_t* q, uint8_t* sb, float* s,
                                   void* stream) {
  if (rows < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 16 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (rows == 0) return NVFP4_SUCCESS;
  if (!s) return NVFP4_ERROR_INVALID_VALUE;
  if (k > 0 && (!x_bf16 || !q || !sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (rows > ((int64_t)1 << 36) || k > ((int64_t)1 << 30)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(amax_in, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  hipStream_t str = (hipStream_t)stream;
  if (k == 0) {
    dim3 grid((unsigned)((rows + 255) / 256));
    if (amax_in)
      hipLaunchKernelGGL(nvfp4::quantize_empty_rows_kernel<nvfp4::MODE_AMAX_IN>, grid, dim3(256), 0,
                         str, rows, amax_in, s);
    else
      hipLaunchKernelGGL(nvfp4::quantize_empty_rows_kernel<nvfp4::MODE_ROW>, grid, dim3(256), 0,
                         str, rows, amax_in, s);
    return nvfp4host::launch_status();
  }
  if (amax_in)
    nvfp4::launch_rows<nvfp4::MODE_AMAX_IN>(x_bf16, rows, k, amax_in, 1, q, sb, s, str);
  else
    nvfp4::launch_rows<nvfp4::MODE_ROW>(x_bf16, rows, k, nullptr, 1, q, sb, s, str);
  return nvfp4host::launch_status();
}

extern "C" int nvfp4_quantize_weight(const uint16_t* w_bf16, int64_t groups, int64_t rows_per_group,
                                     int64_t k, const float* amax_in, float* amax_out, uint8_t* q,
                                     uint8_t* sb, float* s, void* stream) {
  if (groups < 1 || rows_per_group < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 16 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!s || (!amax_in && !amax_out)) return NVFP4_ERROR_INVALID_VALUE;
  const int64_t rows = groups * rows_per_group;
  if (rows > 0 && k > 0 && (!w_bf16 || !q || !sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (groups > ((int64_t)1 << 31) || rows > ((int64_t)1 << 36) || k > ((int64_t)1 << 30))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(amax_in, 4) ||
      !aligned(amax_out, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  hipStream_t str = (hipStream_t)stream;
  const unsigned gsm = (unsigned)((groups + 255) / 256);
  if (!amax_in) {
    hipLaunchKernelGGL(nvfp4::fill_zero_kernel, dim3(gsm < 1024 ? gsm : 1024), dim3(256), 0, str,
                       amax_out, groups);
    const int64_t group_elems = rows_per_group * k;
    if (group_elems > 0) {
      // large chunks (up to 1 MiB of bf16 per block) keep the reads streaming;
      // at least ~1024 blocks keep every CU busy
      const int64_t nvec = group_elems / 8;
      int64_t chunk_vecs = (nvec * groups) / 1024;
      chunk_vecs = chunk_vecs < 4096 ? 4096 : (chunk_vecs > 65536 ? 65536 : chunk_vecs);
      int64_t chunks = (nvec + chunk_vecs - 1) / chunk_vecs;
      if (chunks * groups > ((int64_t)1 << 30)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
      hipLaunchKernelGGL(nvfp4::group_amax_kernel, dim3((unsigned)(chunks * groups)), dim3(256), 0,
                         str, w_bf16, group_elems, chunk_vecs, (int)chunks, amax_out);
    }
  }
  hipLaunchKernelGGL(nvfp4::group_scale_kernel, dim3(gsm), dim3(256), 0, str, groups, amax_in,
                     amax_out, s);
  if (rows > 0 && k > 0)
    nvfp4::launch_rows<nvfp4::MODE_GROUP>(w_bf16, rows, k, amax_in ? amax_in : amax_out,
                                          rows_per_group, q, sb, s, str);
  return nvfp4host::launch_status();
}
