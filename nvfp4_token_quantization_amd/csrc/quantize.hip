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
//    16-byte half-blocks divide evenly); lane j owns half-blocks j, j+L,
//    j+2L, ... (8 elements each) and keeps them in VGPRs, so the row is read
//    from HBM once.  Every load instruction reads L * 16 contiguous bytes.
//  - A block's two halves sit in lanes 2m and 2m+1: each lane takes the
//    packed 16-bit max over its 8 bf16 magnitude bits (exact: non-negative
//    bf16 bit patterns order like their values) and one DPP swap combines
//    the pair, so both lanes hold the block amax.  Of two slots, the even
//    lane derives one block's scale and the odd lane the other's, and a
//    second DPP swap shares the results.
//  - Row amax: DPP / ds_swizzle / readlane max over the row's lanes.
//  - Per row the correctly rounded S = amax / 2688, t = 6 S and 1 / t; per
//    block the correctly rounded a_b / t and 1 / d from fma corrections
//    (block_scale in nvfp4_internal.h); per element one fp32 multiply and
//    half of a gfx950 pack-convert to E2M1 (two elements per instruction).
//    Each lane stores one dword of codes per half-block; even lanes store
//    the scale.
#include "quant_rows.h"
#include "weight_onepass.h"

namespace nvfp4 {

// Grid cap in launched waves per SIMD (4-wave blocks, so also blocks per
// CU); registers allow 4-6 resident, the rest queue behind them.
#ifndef NVFP4_Q_WAVES_PER_SIMD
#define NVFP4_Q_WAVES_PER_SIMD 32
#endif

// One row per L lanes (U half-blocks per lane at most, nh <= L * U); a wave
// handles 64 / L rows per row group and walks row groups with a grid stride,
// loading group i + 1 while it encodes group i (two register buffers,
// unrolled by two so the buffers never move).
template <int L, int U, int MODE>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int nh,
    const float* __restrict__ amax_src, int64_t rows_per_group, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sb, float* __restrict__ s) {
  constexpr int RPW = 64 / L;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int sub = lane / L;
  const int64_t ngroups = (rows + RPW - 1) / RPW;
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t g0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // wave-uniform
  RowData<U> r0, r1;
  if (g0 < ngroups)
    load_rows<L, U, MODE>(x, rows, k, nh, g0 * RPW + sub, j, amax_src, rows_per_group, r0);
  for (; g0 < ngroups; g0 += 2 * stride) {
    const int64_t g1 = g0 + stride, g2 = g1 + stride;
    if (g1 < ngroups)
      load_rows<L, U, MODE>(x, rows, k, nh, g1 * RPW + sub, j, amax_src, rows_per_group, r1);
    encode_rows<L, U, MODE>(r0, rows, k, nh, g0 * RPW + sub, j, amax_src, rows_per_group, q, sb,
                            s);
    if (g2 < ngroups)
      load_rows<L, U, MODE>(x, rows, k, nh, g2 * RPW + sub, j, amax_src, rows_per_group, r0);
    if (g1 < ngroups)
      encode_rows<L, U, MODE>(r1, rows, k, nh, g1 * RPW + sub, j, amax_src, rows_per_group, q,
                              sb, s);
  }
}

// Rows longer than 64 * 16 half-blocks: one wave per row, two passes (the
// second re-reads the row, mostly from L2).
template <int MODE>
__global__ __launch_bounds__(256) void quantize_rows_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int nh,
    const float* __restrict__ amax_src, int64_t rows_per_group, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sb, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * k);
  float amax;
  if (MODE == MODE_ROW) {
    uint32_t rmax = 0;
    for (int h = lane; h < nh; h += 64) rmax = max(rmax, half_amax_bits(xr[h]));
    amax = __uint_as_float(group_max_u32<64>(rmax) << 16);
  } else if (MODE == MODE_AMAX_IN) {
    amax = amax_src[row];
  } else {
    const int64_t gi = row / rows_per_group;
    amax = amax_src[gi];
    if (s && lane == 0 && row == gi * rows_per_group) s[gi] = amax / 2688.0f;
  }
  const RowScale rs = row_scale(amax);
  if (MODE != MODE_GROUP && lane == 0) s[row] = rs.S;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * (k / 2));
  uint8_t* sr = sb + row * (k / 16);
  // nh is even and the stride is even, so lanes 2m and 2m+1 stay together
  // and every lane runs the same number of iterations (DPP needs both).
  for (int h0 = 0; h0 < nh; h0 += 64) {
    const int h = h0 + lane;
    const uint4 a = (h < nh) ? xr[h] : make_uint4(0, 0, 0, 0);
    uint32_t code;
    float inv;
    block_scale(pair_max(half_amax_bits(a)), rs, code, inv);
    if (h < nh) {
      qr[h] = encode_half(a, inv);
      if ((lane & 1) == 0) sr[h >> 1] = (uint8_t)code;
    }
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

// Group amax: block (g, c) of 1024 threads reduces chunk c of group g's
// contiguous elements (4 independent 16-byte streaming loads in flight per
// thread) and folds it into amax[g] with an atomic max on the bit pattern
// (order independent, so the result is deterministic).  Atomics on one
// address serialize (about 10 ns each), so large blocks keep their number
// low for a per-tensor scale (groups = 1) at the same wave count.
__global__ __launch_bounds__(1024) void group_amax_kernel(const uint16_t* __restrict__ w,
                                                          int64_t group_elems, int64_t chunk_vecs,
                                                          int chunks, float* __restrict__ amax) {
  __shared__ uint32_t red[16];
  const int64_t g = blockIdx.x / chunks;
  const int64_t c = blockIdx.x % chunks;
  const int64_t nvec = group_elems / 8;  // 16-byte vectors in the group
  const uint4* base = reinterpret_cast<const uint4*>(w + g * group_elems);
  const int64_t v0 = c * chunk_vecs;
  const int64_t v1 = min(nvec, v0 + chunk_vecs);
  uint32_t m = 0;
  int64_t v = v0 + threadIdx.x;
  for (; v + 3 * 1024 < v1; v += 4 * 1024) {
    uint4 a = ld_stream(base + v), b = ld_stream(base + v + 1024);
    uint4 c2 = ld_stream(base + v + 2048), d = ld_stream(base + v + 3072);
    m = max(m, max(block_amax_bits(a, b), block_amax_bits(c2, d)));
  }
  for (; v < v1; v += 1024) m = max(m, block_amax_bits(base[v], make_uint4(0, 0, 0, 0)));
  m = group_max_u32<64>(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < 16; ++i) r = max(r, red[i]);
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
static RowKernel pick_row_kernel(int nh, int& lanes) {
#define NVFP4_PICK(L)                                                            \
  switch ((nh + L - 1) / L) {                                                    \
    case 1: lanes = L; return quantize_rows_kernel<L, 1, MODE>;                  \
    case 2: lanes = L; return quantize_rows_kernel<L, 2, MODE>;                  \
    case 3: lanes = L; return quantize_rows_kernel<L, 3, MODE>;                  \
    case 4: lanes = L; return quantize_rows_kernel<L, 4, MODE>;                  \
    case 5: lanes = L; return quantize_rows_kernel<L, 5, MODE>;                  \
    case 6: lanes = L; return quantize_rows_kernel<L, 6, MODE>;                  \
    case 7:                                                                      \
    case 8: lanes = L; return quantize_rows_kernel<L, 8, MODE>;                  \
    case 9:                                                                      \
    case 10: lanes = L; return quantize_rows_kernel<L, 10, MODE>;                \
    case 11:                                                                     \
    case 12: lanes = L; return quantize_rows_kernel<L, 12, MODE>;                \
    case 13:                                                                     \
    case 14:                                                                     \
    case 15:                                                                     \
    case 16: lanes = L; return quantize_rows_kernel<L, 16, MODE>;                \
    default: break;                                                              \
  }
  // prefer the widest group that divides the row's half-blocks evenly
  if (nh % 64 == 0 && nh / 64 <= 16) { NVFP4_PICK(64) }
  if (nh % 32 == 0 && nh / 32 <= 16) { NVFP4_PICK(32) }
  if (nh % 16 == 0 && nh / 16 <= 16) { NVFP4_PICK(16) }
  if (nh <= 16 * 16 && nh < 32) { NVFP4_PICK(16) }
  if (nh <= 32 * 16 && nh < 64) { NVFP4_PICK(32) }
  if (nh <= 64 * 16) { NVFP4_PICK(64) }
#undef NVFP4_PICK
  lanes = 0;
  return nullptr;
}

template <int MODE>
static void launch_rows(const uint16_t* x, int64_t rows, int64_t k, const float* amax_src,
                        int64_t rows_per_group, uint8_t* q, uint8_t* sb, float* s,
                        hipStream_t stream) {
  const int nh = (int)(k / 8);  // 16-byte half-blocks per row
  int lanes = 0;
  RowKernel kern = pick_row_kernel<MODE>(nh, lanes);
  if (kern) {
    // a few row groups per wave at the largest shapes (loads of group i + 1
    // overlap the encoding of group i), and enough queued waves that one
    // wave's loads overlap another's arithmetic at the small ones
    const int64_t rows_per_block = 4 * (64 / lanes);
    const int64_t need = (rows + rows_per_block - 1) / rows_per_block;
    const int64_t cap = (int64_t)nvfp4host::num_cus() * NVFP4_Q_WAVES_PER_SIMD;
    dim3 grid((unsigned)(need < cap ? need : cap));
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, x, rows, k, nh, amax_src,
                       rows_per_group, q, sb, s);
  } else {
    dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(quantize_rows_long_kernel<MODE>, grid, dim3(256), 0, stream, x, rows, k,
                       nh, amax_src, rows_per_group, q, sb, s);
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
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.bf16_finite(x_bf16, rows * k);
    chk.f32_finite(amax_in, rows, true);
    if ((st = chk.result())) return st;
  }
#endif
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
  // amax_out is written while s is (the reduction target, then the scales)
  if (amax_out && amax_out < s + groups && s < amax_out + groups) return NVFP4_ERROR_INVALID_VALUE;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.bf16_finite(w_bf16, rows * k);
    chk.f32_finite(amax_in, groups, true);
    if ((st = chk.result())) return st;
  }
#endif
  hipStream_t str = (hipStream_t)stream;
  // one HBM pass when each group is large enough and a team of workgroups
  // holds it in registers (weight_onepass.h)
  if (!amax_in && rows > 0 && k > 0 &&
      nvfp4::launch_weight_onepass(w_bf16, groups, rows_per_group, k, amax_out, q, sb, s,
                                   nvfp4::OP_LIMIT_MS, nvfp4::OP_MIN_GROUP_BYTES, nvfp4::OP_MIN_TEAMS, str))
    return nvfp4host::launch_status();
  const unsigned gsm = (unsigned)((groups + 255) / 256);
  if (!amax_in) {
    hipLaunchKernelGGL(nvfp4::fill_zero_kernel, dim3(gsm < 1024 ? gsm : 1024), dim3(256), 0, str,
                       amax_out, groups);
    const int64_t group_elems = rows_per_group * k;
    if (group_elems > 0) {
      // large chunks (256 KiB to 4 MiB of bf16 per block) keep the reads
      // streaming; about 256 blocks of 16 waves keep every CU busy
      const int64_t nvec = group_elems / 8;
      int64_t chunk_vecs = (nvec * groups) / 256;
      chunk_vecs = chunk_vecs < 16384 ? 16384 : (chunk_vecs > 262144 ? 262144 : chunk_vecs);
      int64_t chunks = (nvec + chunk_vecs - 1) / chunk_vecs;
      if (chunks * groups > ((int64_t)1 << 30)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
      hipLaunchKernelGGL(nvfp4::group_amax_kernel, dim3((unsigned)(chunks * groups)), dim3(1024), 0,
                         str, w_bf16, group_elems, chunk_vecs, (int)chunks, amax_out);
    }
  }
  // the encode pass stores S[g] itself, except when it does not run or the
  // amax was supplied (then amax_out also receives a copy of amax_in)
  const bool enc = rows > 0 && k > 0;
  const bool s_in_enc = enc && !amax_in;
  if (!s_in_enc)
    hipLaunchKernelGGL(nvfp4::group_scale_kernel, dim3(gsm), dim3(256), 0, str, groups, amax_in,
                       amax_out, s);
  if (enc)
    nvfp4::launch_rows<nvfp4::MODE_GROUP>(w_bf16, rows, k, amax_in ? amax_in : amax_out,
                                          rows_per_group, q, sb, s_in_enc ? s : nullptr, str);
  return nvfp4host::launch_status();
}
