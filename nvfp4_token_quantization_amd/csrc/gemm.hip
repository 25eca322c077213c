// gemm.hip -- dense and grouped (MoE) block-scaled W4A4 GEMM for gfx950.
//
// Y[m, n] = S_A[m] * S_B * sum_k u_A[m, k] * u_B[n, k],  u = s_b * e2m1(q)
// (the Miles page, section 速读: X ~ s_token * s_block * X_FP4; the per-token
// scale is applied in the epilogue, as that page's 实验结果 item 10 says a
// fused kernel should).  Grouped: expert g owns output rows
// [offsets[g], offsets[g+1]) of a contiguous per-expert layout whose offsets
// stay on the device ("miniTE报告", section Transformer Engine路径优化).
//
// Why not gfx950's scaled MFMA: it takes one power-of-two (E8M0) scale per
// 32 K-elements, while NVFP4 has an E4M3 scale per 16.  Instead each unit u
// is decoded exactly into fp16: u has at most 6 significant bits and lies in
// [2^-10, 2688], so fp16 holds it exactly, and so do the products in the fp32
// accumulator.  fp16 (not bf16) is used because gfx950 has a packed fp16
// multiply to apply the block scale; the MFMA rate is the same.
//
// Decode of 8 elements (one MFMA operand, one dword of packed codes):
//   4 x v_cvt_scalef32_pk_f16_fp4 with scale 2^8 -> e2m1 * 256 (exact; the
//       converter applies only the exponent of its scale)
//   4 x v_pk_mul_f16 by h = fp16 bit pattern (code << 7), which is exactly
//       s_b * 2^-8 (E4M3's 4+3 bits land on fp16's exponent and mantissa with
//       a bias difference of 8, subnormal codes included)
//   product = e2m1 * s_b = u, exact and normal in fp16.
//
// Tiling: 256 threads = 2 x 2 waves, each wave owns TM x TN tiles of 32 x 32
// (v_mfma_f32_32x32x16_f16).  A K stage is 128 elements: per row 64 bytes
// of codes and 8 scale bytes, staged in LDS (double buffered, rows padded to
// avoid bank conflicts).  Lane group h = lane / 32 of a wave takes the K
// elements [64h, 64h+64) of the stage for both A and B; the MFMA's K order
// inside a stage is therefore a permutation, identical for A and B, which
// leaves the dot products unchanged.
#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int BK = 128;          // K elements per stage
constexpr int ROWB = BK / 2;     // code bytes per row per stage
constexpr int SROW = 80;         // LDS row stride for codes (64 + 16 pad)
constexpr int SCB = BK / 16;     // scale bytes per row per stage
constexpr int MAX_GROUPS = 1024;

struct GemmArgs {
  const uint8_t* a_q;
  const uint8_t* a_sb;
  const float* a_s;
  int64_t a_rows;
  const int32_t* row_index;  // grouped only (nullable)
  int64_t m_total;           // grouped: output rows; dense: m
  const int32_t* offsets;    // grouped only
  int groups;                // grouped only
  const uint8_t* b_q;
  const uint8_t* b_sb;
  const float* b_s;
  int64_t n, k;
  float* y;
  int tiles_n;
};

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// 8 decoded fp16 units from one dword of codes and a (h, h) scale pair
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16x2 sc) {
  f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0));
  f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1));
  f16x2 p2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2));
  f16x2 p3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3));
  p0 = p0 * sc;
  p1 = p1 * sc;
  p2 = p2 * sc;
  p3 = p3 * sc;
  return (f16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// (code << 7, code << 7) as an fp16 pair: s_b * 2^-8 in both halves
__device__ __forceinline__ f16x2 scale_pair(uint32_t scales4, int blk) {
  uint32_t c = (scales4 >> (8 * blk)) & 0xFFu;
  return as_h2((c << 7) | (c << 23));
}

// Global -> register staging of one K stage for BM rows of A and BN rows of B.
template <int BM, int BN, bool FAST>
struct Stage {
  static constexpr int ACH = BM * 4 / 256;  // 16-byte chunks of codes per thread (A)
  static constexpr int BCH = BN * 4 / 256;
  uint4 a[ACH];
  uint4 b[BCH];
  uint2 as;  // 8 scale bytes of one A row (threads < BM)
  uint2 bs;  // 8 scale bytes of one B row (threads < BN)
};

// Row pointers of the tile, computed once per tile.
template <int BM, int BN>
struct TileRows {
  int64_t arow[BM * 4 / 256];  // A source row per code chunk (-1: zero)
  int64_t brow[BN * 4 / 256];
  int64_t arow_s;              // A source row for the scale bytes (threads < BM)
  int64_t brow_s;
};

// 8-byte load of bytes [off, off + 8) of a row with `valid` bytes (K tail):
// bytes past `valid` read as zero and are never fetched.  `row + off` must be
// 8-byte aligned when the 8 bytes are all valid.
__device__ __forceinline__ uint2 load8_masked(const uint8_t* row, int64_t off, int64_t valid) {
  if (off + 8 <= valid) return *reinterpret_cast<const uint2*>(row + off);
  uint32_t v[2] = {0u, 0u};
  for (int i = 0; i < 8; ++i)
    if (off + i < valid) v[i >> 2] |= (uint32_t)row[off + i] << (8 * (i & 3));
  return make_uint2(v[0], v[1]);
}

// Same with byte loads only (scale rows of k/16 bytes need not be aligned).
__device__ __forceinline__ uint2 load8_bytes(const uint8_t* row, int64_t off, int64_t valid) {
  uint32_t v[2] = {0u, 0u};
  for (int i = 0; i < 8; ++i)
    if (off + i < valid) v[i >> 2] |= (uint32_t)row[off + i] << (8 * (i & 3));
  return make_uint2(v[0], v[1]);
}

template <int BM, int BN, bool FAST>
__device__ __forceinline__ void load_stage(const GemmArgs& p, const TileRows<BM, BN>& tr,
                                           const uint8_t* bq_base, const uint8_t* bsb_base,
                                           int64_t k0, Stage<BM, BN, FAST>& st) {
  const int tid = threadIdx.x;
  const int64_t rowb = p.k / 2;    // code bytes per row
  const int64_t rows_s = p.k / 16;  // scale bytes per row
  const int part = tid & 3;         // which 16-byte chunk of the 64-byte stage row
  const int64_t off = k0 / 2 + part * 16;
#pragma unroll
  for (int i = 0; i < Stage<BM, BN, FAST>::ACH; ++i) {
    const int64_t r = tr.arow[i];
    if (r < 0) {
      st.a[i] = make_uint4(0, 0, 0, 0);
    } else if (FAST) {
      st.a[i] = *reinterpret_cast<const uint4*>(p.a_q + r * rowb + off);
    } else {
      const uint8_t* rp = p.a_q + r * rowb;
      uint2 lo = load8_masked(rp, off, rowb), hi = load8_masked(rp, off + 8, rowb);
      st.a[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
#pragma unroll
  for (int i = 0; i < Stage<BM, BN, FAST>::BCH; ++i) {
    const int64_t r = tr.brow[i];
    if (r < 0) {
      st.b[i] = make_uint4(0, 0, 0, 0);
    } else if (FAST) {
      st.b[i] = *reinterpret_cast<const uint4*>(bq_base + r * rowb + off);
    } else {
      const uint8_t* rp = bq_base + r * rowb;
      uint2 lo = load8_masked(rp, off, rowb), hi = load8_masked(rp, off + 8, rowb);
      st.b[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  const int64_t soff = k0 / 16;
  if (tid < BM) {
    if (tr.arow_s < 0) st.as = make_uint2(0, 0);
    else if (FAST) st.as = *reinterpret_cast<const uint2*>(p.a_sb + tr.arow_s * rows_s + soff);
    else st.as = load8_bytes(p.a_sb + tr.arow_s * rows_s, soff, rows_s);
  }
  if (tid < BN) {
    if (tr.brow_s < 0) st.bs = make_uint2(0, 0);
    else if (FAST) st.bs = *reinterpret_cast<const uint2*>(bsb_base + tr.brow_s * rows_s + soff);
    else st.bs = load8_bytes(bsb_base + tr.brow_s * rows_s, soff, rows_s);
  }
}

template <int BM, int BN, bool FAST>
__device__ __forceinline__ void store_stage(const Stage<BM, BN, FAST>& st, uint8_t* sA, uint8_t* sB,
                                            uint8_t* sAs, uint8_t* sBs) {
  const int tid = threadIdx.x;
  const int part = tid & 3;
#pragma unroll
  for (int i = 0; i < Stage<BM, BN, FAST>::ACH; ++i) {
    const int row = (tid + 256 * i) >> 2;
    *reinterpret_cast<uint4*>(sA + row * SROW + part * 16) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < Stage<BM, BN, FAST>::BCH; ++i) {
    const int row = (tid + 256 * i) >> 2;
    *reinterpret_cast<uint4*>(sB + row * SROW + part * 16) = st.b[i];
  }
  if (tid < BM) *reinterpret_cast<uint2*>(sAs + tid * SCB) = st.as;
  if (tid < BN) *reinterpret_cast<uint2*>(sBs + tid * SCB) = st.bs;
}

template <int TM, int TN, bool FAST>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  constexpr int WM = 32 * TM, WN = 32 * TN;
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int A_BYTES = BM * SROW, B_BYTES = BN * SROW;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES + (BM + BN) * SCB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];
  __shared__ int32_t s_prefix[MAX_GROUPS + 1];
  __shared__ int32_t s_wsum[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;   // K half of the stage this lane feeds
  const int li = lane & 31;  // row (A) / column (B) inside a 32-slab

  // ---- tile -> (group, rows, n0)
  int64_t mt, row_lo, row_hi;
  int g = 0;
  const int64_t tile = blockIdx.x;
  const int64_t nt = tile % p.tiles_n;
  mt = tile / p.tiles_n;
  if (p.offsets) {
    // per-group m-tile counts and their exclusive prefix, from device offsets
    const int G = p.groups;
    int32_t local = 0;
    int32_t cnt[MAX_GROUPS / 256];
#pragma unroll
    for (int i = 0; i < MAX_GROUPS / 256; ++i) {
      const int gg = tid * (MAX_GROUPS / 256) + i;
      int32_t c = 0;
      if (gg < G) {
        int64_t lo = min(max((int64_t)p.offsets[gg], (int64_t)0), p.m_total);
        int64_t hi = min(max((int64_t)p.offsets[gg + 1], lo), p.m_total);
        c = (int32_t)((hi - lo + BM - 1) / BM);
      }
      cnt[i] = c;
      local += c;
    }
    // block-wide exclusive scan of `local`
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int32_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    int32_t run = base + incl - local;
#pragma unroll
    for (int i = 0; i < MAX_GROUPS / 256; ++i) {
      const int gg = tid * (MAX_GROUPS / 256) + i;
      if (gg <= G) s_prefix[gg] = run;
      run += cnt[i];
    }
    __syncthreads();
    const int32_t total_mt = s_prefix[G];
    if (mt >= total_mt) return;  // block-uniform
    // binary search: largest g with s_prefix[g] <= mt
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int64_t glo = min(max((int64_t)p.offsets[g], (int64_t)0), p.m_total);
    const int64_t ghi = min(max((int64_t)p.offsets[g + 1], glo), p.m_total);
    row_lo = glo + (mt - s_prefix[g]) * BM;
    row_hi = min(ghi, row_lo + BM);
  } else {
    row_lo = mt * BM;
    row_hi = min(p.m_total, row_lo + BM);
  }
  const int64_t n0 = nt * BN;
  const uint8_t* bq_base = p.b_q + (int64_t)g * p.n * (p.k / 2);
  const uint8_t* bsb_base = p.b_sb + (int64_t)g * p.n * (p.k / 16);

  auto a_source = [&](int64_t out_row) -> int64_t {
    if (out_row >= row_hi) return -1;
    int64_t r = p.row_index ? (int64_t)p.row_index[out_row] : out_row;
    return (r >= 0 && r < p.a_rows) ? r : -1;
  };

  TileRows<BM, BN> tr;
#pragma unroll
  for (int i = 0; i < BM * 4 / 256; ++i) tr.arow[i] = a_source(row_lo + ((tid + 256 * i) >> 2));
#pragma unroll
  for (int i = 0; i < BN * 4 / 256; ++i) {
    const int64_t c = n0 + ((tid + 256 * i) >> 2);
    tr.brow[i] = c < p.n ? c : -1;
  }
  tr.arow_s = tid < BM ? a_source(row_lo + tid) : -1;
  tr.brow_s = (tid < BN && n0 + tid < p.n) ? n0 + tid : -1;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){0};

  const int64_t nstages = (p.k + BK - 1) / BK;
  Stage<BM, BN, FAST> st;
  if (nstages > 0) {
    load_stage<BM, BN, FAST>(p, tr, bq_base, bsb_base, 0, st);
    uint8_t* s0 = smem;
    store_stage<BM, BN, FAST>(st, s0, s0 + A_BYTES, s0 + A_BYTES + B_BYTES,
                              s0 + A_BYTES + B_BYTES + BM * SCB);
  }
  __syncthreads();

  for (int64_t s = 0; s < nstages; ++s) {
    uint8_t* cur = smem + (s & 1) * STAGE_BYTES;
    uint8_t* nxt = smem + ((s + 1) & 1) * STAGE_BYTES;
    const bool more = s + 1 < nstages;
    if (more) load_stage<BM, BN, FAST>(p, tr, bq_base, bsb_base, (s + 1) * BK, st);

    const uint8_t* sA = cur;
    const uint8_t* sB = cur + A_BYTES;
    const uint8_t* sAs = cur + A_BYTES + B_BYTES;
    const uint8_t* sBs = sAs + BM * SCB;
    // this lane's 32 code bytes and 4 scale bytes per slab
    uint4 ra[TM][2], rb[TN][2];
    uint32_t sa4[TM], sb4[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + 32 * i + li;
      const uint4* pa = reinterpret_cast<const uint4*>(sA + row * SROW + 32 * h);
      ra[i][0] = pa[0];
      ra[i][1] = pa[1];
      sa4[i] = *reinterpret_cast<const uint32_t*>(sAs + row * SCB + 4 * h);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WN + 32 * j + li;
      const uint4* pb = reinterpret_cast<const uint4*>(sB + row * SROW + 32 * h);
      rb[j][0] = pb[0];
      rb[j][1] = pb[1];
      sb4[j] = *reinterpret_cast<const uint32_t*>(sBs + row * SCB + 4 * h);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint4& v = ra[i][t >> 2];
        const uint32_t w = (t & 3) == 0 ? v.x : (t & 3) == 1 ? v.y : (t & 3) == 2 ? v.z : v.w;
        fa[i] = decode8(w, scale_pair(sa4[i], t >> 1));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint4& v = rb[j][t >> 2];
        const uint32_t w = (t & 3) == 0 ? v.x : (t & 3) == 1 ? v.y : (t & 3) == 2 ? v.z : v.w;
        fb[j] = decode8(w, scale_pair(sb4[j], t >> 1));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more)
      store_stage<BM, BN, FAST>(st, nxt, nxt + A_BYTES, nxt + A_BYTES + B_BYTES,
                                nxt + A_BYTES + B_BYTES + BM * SCB);
    __syncthreads();
  }

  // ---- epilogue: Y = acc * (S_A[row] * S_B)
  const float sbw = p.b_s[g];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row_lo + wm * WM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= row_hi) continue;
      const int64_t ar = a_source(row);
      const float sc = (ar >= 0 ? p.a_s[ar] : 0.0f) * sbw;
      float* yr = p.y + row * p.n;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * WN + 32 * j + li;
        if (col < p.n) yr[col] = acc[i][j][r] * sc;
      }
    }
  }
}

template <int TM, int TN>
static void launch_gemm(const GemmArgs& a, int64_t tiles_m, hipStream_t stream) {
  constexpr int BN = 64 * TN;
  GemmArgs p = a;
  p.tiles_n = (int)((p.n + BN - 1) / BN);
  const int64_t blocks = tiles_m * p.tiles_n;
  const bool fast = (p.k % BK) == 0 && nvfp4host::aligned(p.a_q, 16) &&
                    nvfp4host::aligned(p.b_q, 16) && nvfp4host::aligned(p.a_sb, 8) &&
                    nvfp4host::aligned(p.b_sb, 8);
  if (fast)
    hipLaunchKernelGGL((gemm_kernel<TM, TN, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<TM, TN, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
}

// Y = 0 for k == 0 (no operand bytes to read).
__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ y, int64_t n_elems) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_elems; i += (int64_t)gridDim.x * 256)
    y[i] = 0.0f;
}

constexpr int TM_DEF = 2, TN_DEF = 2;
constexpr int BM_DEF = 64 * TM_DEF;

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s, int64_t m,
                          const uint8_t* b_q, const uint8_t* b_sb, const float* b_s, int64_t n,
                          int64_t k, float* y, void* stream) {
  if (m < 0 || n < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 16 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (m == 0 || n == 0) return NVFP4_SUCCESS;
  if (!y || !a_s || !b_s) return NVFP4_ERROR_INVALID_VALUE;
  if (k > 0 && (!a_q || !a_sb || !b_q || !b_sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (m > ((int64_t)1 << 31) || n > ((int64_t)1 << 31) || k > ((int64_t)1 << 24))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_sb, 16) || !aligned(b_sb, 16) ||
      !aligned(y, 16) || !aligned(a_s, 4) || !aligned(b_s, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  hipStream_t str = (hipStream_t)stream;
  if (k == 0) {
    hipLaunchKernelGGL(nvfp4::zero_rows_kernel, dim3(1024), dim3(256), 0, str, y, m * n);
    return nvfp4host::launch_status();
  }
  nvfp4::GemmArgs p{};
  p.a_q = a_q; p.a_sb = a_sb; p.a_s = a_s; p.a_rows = m;
  p.row_index = nullptr; p.m_total = m; p.offsets = nullptr; p.groups = 1;
  p.b_q = b_q; p.b_sb = b_sb; p.b_s = b_s; p.n = n; p.k = k; p.y = y;
  const int64_t tiles_m = (m + nvfp4::BM_DEF - 1) / nvfp4::BM_DEF;
  nvfp4::launch_gemm<nvfp4::TM_DEF, nvfp4::TN_DEF>(p, tiles_m, str);
  return nvfp4host::launch_status();
}

extern "C" int nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s,
                                  int64_t a_rows, const int32_t* row_index, int64_t m_total,
                                  const int32_t* offsets, int64_t groups, const uint8_t* b_q,
                                  const uint8_t* b_sb, const float* b_s, int64_t n, int64_t k,
                                  float* y, void* stream) {
  if (groups < 1 || a_rows < 0 || m_total < 0 || n < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 16 != 0 || groups > nvfp4::MAX_GROUPS) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (m_total == 0 || n == 0) return NVFP4_SUCCESS;
  if (!offsets || !y || !b_s || (a_rows > 0 && !a_s)) return NVFP4_ERROR_INVALID_VALUE;
  if (!row_index && a_rows < m_total) return NVFP4_ERROR_INVALID_VALUE;
  if (k > 0 && a_rows > 0 && (!a_q || !a_sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (k > 0 && (!b_q || !b_sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (m_total > ((int64_t)1 << 31) || a_rows > ((int64_t)1 << 31) || n > ((int64_t)1 << 31) ||
      k > ((int64_t)1 << 24))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_sb, 16) || !aligned(b_sb, 16) ||
      !aligned(y, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(offsets, 4) ||
      !aligned(row_index, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  hipStream_t str = (hipStream_t)stream;
  nvfp4::GemmArgs p{};
  p.a_q = a_q; p.a_sb = a_sb; p.a_s = a_s; p.a_rows = a_rows;
  p.row_index = row_index; p.m_total = m_total; p.offsets = offsets; p.groups = (int)groups;
  p.b_q = b_q; p.b_sb = b_sb; p.b_s = b_s; p.n = n; p.k = k; p.y = y;
  // upper bound on m-tiles without reading offsets: each group adds at most
  // one partial tile
  const int64_t tiles_m = (m_total + nvfp4::BM_DEF - 1) / nvfp4::BM_DEF + groups;
  // k == 0 needs no special case: the K loop is empty and the epilogue writes
  // zeros to exactly the rows the groups own
  nvfp4::launch_gemm<nvfp4::TM_DEF, nvfp4::TN_DEF>(p, tiles_m, str);
  return nvfp4host::launch_status();
}
