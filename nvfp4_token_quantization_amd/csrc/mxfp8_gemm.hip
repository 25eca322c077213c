// mxfp8_gemm.hip -- dense and grouped (MoE) MXFP8 GEMM on gfx950's scaled
// MFMA: Y[m, n] = sum over 32-blocks of 2^(e_A + e_B) * sum_32 a * b, fp32
// accumulate and output.
//
// MXFP8 (Miles page, section MXFP8格式背景: 32 E4M3 values per E8M0 scale)
// maps onto v_mfma_scale_f32_32x32x64_f8f6f4 directly: the instruction takes
// one E8M0 scale per row (A) / column (B) per 32 K-elements.  Its operand
// layout, measured on MI355X: lane (li, h) supplies 32 bytes for row li
// (A) or column li (B), bytes 0..15 from the MFMA's first 32-block and 16..31
// from its second, the two lane halves h = 0, 1 splitting each block; the
// scale of (row li, block b) comes from lane li + 32 b.  Which K positions a
// byte stands for inside a block does not matter as long as A and B agree,
// so lane (li, h) simply reads bytes [32 b + 16 h, +16) of each block b.
//
// Tiling follows the NVFP4 kernel (register-direct, one wave per block, a
// 128 x 128 tile of 4 x 4 MFMA tiles with 256 fp32 accumulators, operands
// loaded from L2 one K stage of 64 ahead into a register double buffer, the
// XCD-aware tile order of tile_sched.h), without any decode: the E4M3 bytes
// and E8M0 codes go to the MFMA as they are stored.
#include "tile_sched.h"

namespace nvfp4 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int MX_BK = 64;  // K elements per stage (one MFMA K step, two blocks)

struct MxGemmArgs {
  const uint8_t* a_q;
  const uint8_t* a_sc;
  int64_t a_rows;
  const int32_t* row_index;  // grouped only (nullable)
  const uint8_t* b_q;
  const uint8_t* b_sc;
  int64_t n, k;
  float* y;
  TileGrid t;
};

template <int TM, int TN>
struct MxStage {
  uint4 a[TM][2];
  uint4 b[TN][2];
  uint32_t as[TM];
  uint32_t bs[TN];
};

// 16 bytes [off, off + 16) of a row holding `valid` bytes (bytes past the
// end read as zero and are not fetched)
__device__ __forceinline__ uint4 mx_load16(const uint8_t* row, int64_t off, int64_t valid,
                                           bool fast) {
  if (fast || off + 16 <= valid) return *reinterpret_cast<const uint4*>(row + off);
  if (off >= valid) return make_uint4(0, 0, 0, 0);
  uint32_t v[4] = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 16; ++i)
    if (off + i < valid) v[i >> 2] |= (uint32_t)row[off + i] << (8 * (i & 3));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Operand rows are kept as 32-bit row numbers (the register file is full):
// rows outside the operand (ragged tiles, bad row indices) use row 0 of B,
// which exists whenever there is K work, so every load is in bounds and
// branch-free; a clear mask bit replaces their data by zeros (scale 2^0).
template <int TM, int TN, int VS, bool FAST>
__device__ __forceinline__ void mx_load(const MxGemmArgs& p, const uint8_t* aq, const uint8_t* asc,
                                        const uint32_t* arow, uint32_t amask, const uint8_t* bq,
                                        const uint8_t* bsc, const uint32_t* brow, uint32_t bmask,
                                        int h, int64_t k0, MxStage<TM, TN>& r) {
  const int64_t nblk = p.k / 32;
  const int64_t blk = k0 / 32 + h;  // the block whose scale this lane supplies
  const bool blk_ok = FAST || blk < nblk;
  const int64_t o0 = k0 + 16 * h, o1 = k0 + 32 + 16 * h;
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    const bool ok = (amask >> i) & 1u;
    const uint8_t* rq = (ok ? aq : p.b_q) + (int64_t)arow[i] * p.k;
    const uint8_t* rs = (ok ? asc : p.b_sc) + (int64_t)arow[i] * nblk;
    const uint4 x0 = mx_load16(rq, o0, p.k, FAST);
    const uint4 x1 = mx_load16(rq, o1, p.k, FAST);
    const uint32_t sc = blk_ok ? (uint32_t)rs[blk_ok ? blk : 0] : 127u;
    r.a[i][0] = ok ? x0 : z;
    r.a[i][1] = ok ? x1 : z;
    r.as[i] = ok ? sc : 127u;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const bool ok = (bmask >> j) & 1u;
    const uint8_t* rq = (ok ? bq : p.b_q) + (int64_t)brow[j] * p.k;
    const uint8_t* rs = (ok ? bsc : p.b_sc) + (int64_t)brow[j] * nblk;
    const uint4 x0 = mx_load16(rq, o0, p.k, FAST);
    const uint4 x1 = mx_load16(rq, o1, p.k, FAST);
    const uint32_t sc = blk_ok ? (uint32_t)rs[blk_ok ? blk : 0] : 127u;
    r.b[j][0] = ok ? x0 : z;
    r.b[j][1] = ok ? x1 : z;
    r.bs[j] = ok ? sc : 127u;
  }
}

__device__ __forceinline__ i32x8 mx_operand(const uint4& lo, const uint4& hi) {
  return (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int TM, int TN, int VS>
__device__ __forceinline__ void mx_compute(const MxStage<TM, TN>& r, f32x16 (&acc)[TM][TN]) {
  i32x8 fa[TM], fb[TN];
#pragma unroll
  for (int i = 0; i < VS; ++i) fa[i] = mx_operand(r.a[i][0], r.a[i][1]);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb[j] = mx_operand(r.b[j][0], r.b[j][1]);
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fa[i], fb[j], acc[i][j], 0, 0, 0, (int)r.as[i], 0, (int)r.bs[j]);
}

template <int TM, int TN, int VS, bool FAST>
__device__ __forceinline__ void mx_body(const MxGemmArgs& p, const uint8_t* bq,
                                        const uint8_t* bsc, const uint32_t* arow, uint32_t amask,
                                        const uint32_t* brow, uint32_t bmask, int h, int li,
                                        int64_t row_lo, int64_t row_hi, int64_t n0) {
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){0};
  const int64_t nstages = (p.k + MX_BK - 1) / MX_BK;
  MxStage<TM, TN> r0, r1;
  if (nstages > 0) mx_load<TM, TN, VS, FAST>(p, p.a_q, p.a_sc, arow, amask, bq, bsc, brow, bmask, h, 0, r0);
  int64_t s = 0;
  for (; s + 1 < nstages; s += 2) {
    mx_load<TM, TN, VS, FAST>(p, p.a_q, p.a_sc, arow, amask, bq, bsc, brow, bmask, h, (s + 1) * MX_BK, r1);
    mx_compute<TM, TN, VS>(r0, acc);
    if (s + 2 < nstages) mx_load<TM, TN, VS, FAST>(p, p.a_q, p.a_sc, arow, amask, bq, bsc, brow, bmask, h, (s + 2) * MX_BK, r0);
    mx_compute<TM, TN, VS>(r1, acc);
  }
  if (s < nstages) mx_compute<TM, TN, VS>(r0, acc);
#pragma unroll
  for (int i = 0; i < VS; ++i) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int64_t row = row_lo + 32 * i + 8 * (rr >> 2) + 4 * h + (rr & 3);
      if (row >= row_hi) continue;
      float* yr = p.y + row * p.n;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + 32 * j + li;
        if (col < p.n) yr[col] = acc[i][j][rr];
      }
    }
  }
}

template <int TM, int TN, bool FAST>
__global__ __launch_bounds__(64) void mxfp8_gemm_kernel(MxGemmArgs p) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  __shared__ int32_t s_prefix[MAX_GROUPS + 1];
  const int lane = threadIdx.x;
  const int h = lane >> 5, li = lane & 31;
  TileRange tr;
  if (!schedule_tile<BM, BN>(p.t, lane, s_prefix, tr)) return;  // block-uniform
  const int64_t row_lo = tr.row_lo, row_hi = tr.row_hi, n0 = tr.n0;
  const uint8_t* bq_base = p.b_q + (int64_t)tr.g * p.n * p.k;
  const uint8_t* bsc_base = p.b_sc + (int64_t)tr.g * p.n * (p.k / 32);
  uint32_t arow[TM], brow[TN];
  uint32_t amask = 0, bmask = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t orow = row_lo + 32 * i + li;
    int64_t r = -1;
    if (orow < row_hi) {
      r = p.row_index ? (int64_t)p.row_index[orow] : orow;
      if (r < 0 || r >= p.a_rows) r = -1;
    }
    arow[i] = r >= 0 ? (uint32_t)r : 0u;
    amask |= (r >= 0 ? 1u : 0u) << i;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t c = n0 + 32 * j + li;
    brow[j] = c < p.n ? (uint32_t)c : 0u;
    bmask |= (c < p.n ? 1u : 0u) << j;
  }
  const int vslabs = (int)min((int64_t)TM, (row_hi - row_lo + 31) / 32);
  static_assert(TM == 4, "slab dispatch is written for TM == 4");
  switch (vslabs) {
    case 4: mx_body<TM, TN, 4, FAST>(p, bq_base, bsc_base, arow, amask, brow, bmask, h, li, row_lo, row_hi, n0); break;
    case 3: mx_body<TM, TN, 3, FAST>(p, bq_base, bsc_base, arow, amask, brow, bmask, h, li, row_lo, row_hi, n0); break;
    case 2: mx_body<TM, TN, 2, FAST>(p, bq_base, bsc_base, arow, amask, brow, bmask, h, li, row_lo, row_hi, n0); break;
    default: mx_body<TM, TN, 1, FAST>(p, bq_base, bsc_base, arow, amask, brow, bmask, h, li, row_lo, row_hi, n0); break;
  }
}

static void launch_mx(const MxGemmArgs& a, bool grouped, hipStream_t stream) {
  MxGemmArgs p = a;
  const int64_t blocks = plan_tiles<128, 128>(p.t, p.n, grouped);
  const bool fast = (p.k % MX_BK) == 0;  // rows are 16-byte aligned since k % 32 == 0
  if (fast)
    hipLaunchKernelGGL((mxfp8_gemm_kernel<4, 4, true>), dim3((unsigned)blocks), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((mxfp8_gemm_kernel<4, 4, false>), dim3((unsigned)blocks), dim3(64), 0, stream, p);
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_mxfp8_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t m,
                                const uint8_t* b_q, const uint8_t* b_sc, int64_t n, int64_t k,
                                float* y, void* stream) {
  if (m < 0 || n < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 32 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (m == 0 || n == 0) return NVFP4_SUCCESS;
  if (!y || (k > 0 && (!a_q || !a_sc || !b_q || !b_sc))) return NVFP4_ERROR_INVALID_VALUE;
  if (m > ((int64_t)1 << 31) || n > ((int64_t)1 << 31) || k > ((int64_t)1 << 24))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(y, 16)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  nvfp4::MxGemmArgs p{};
  p.a_q = a_q; p.a_sc = a_sc; p.a_rows = m; p.row_index = nullptr;
  p.b_q = b_q; p.b_sc = b_sc; p.n = n; p.k = k; p.y = y;
  p.t.m_total = m; p.t.offsets = nullptr; p.t.groups = 1;
  nvfp4::launch_mx(p, false, (hipStream_t)stream);
  return nvfp4host::launch_status();
}

extern "C" int nvfp4_mxfp8_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t a_rows,
                                        const int32_t* row_index, int64_t m_total,
                                        const int32_t* offsets, int64_t groups,
                                        const uint8_t* b_q, const uint8_t* b_sc, int64_t n,
                                        int64_t k, float* y, void* stream) {
  if (groups < 1 || a_rows < 0 || m_total < 0 || n < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 32 != 0 || groups > nvfp4::MAX_GROUPS) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (m_total == 0 || n == 0) return NVFP4_SUCCESS;
  if (!offsets || !y) return NVFP4_ERROR_INVALID_VALUE;
  if (!row_index && a_rows < m_total) return NVFP4_ERROR_INVALID_VALUE;
  if (k > 0 && a_rows > 0 && (!a_q || !a_sc)) return NVFP4_ERROR_INVALID_VALUE;
  if (k > 0 && (!b_q || !b_sc)) return NVFP4_ERROR_INVALID_VALUE;
  if (m_total > ((int64_t)1 << 31) || a_rows > ((int64_t)1 << 31) || n > ((int64_t)1 << 31) ||
      k > ((int64_t)1 << 24))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(y, 16) || !aligned(offsets, 4) ||
      !aligned(row_index, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  nvfp4::MxGemmArgs p{};
  p.a_q = a_q; p.a_sc = a_sc; p.a_rows = a_rows; p.row_index = row_index;
  p.b_q = b_q; p.b_sc = b_sc; p.n = n; p.k = k; p.y = y;
  p.t.m_total = m_total; p.t.offsets = offsets; p.t.groups = (int)groups;
  nvfp4::launch_mx(p, true, (hipStream_t)stream);
  return nvfp4host::launch_status();
}
