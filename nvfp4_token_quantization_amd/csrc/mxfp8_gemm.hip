// mxfp8_gemm.hip -- entry points of the dense and grouped (MoE) MXFP8 GEMM
// (gfx950): Y[m, n] = sum over 32-blocks of 2^(e_A + e_B) * sum_32 a * b,
// with every product formed exactly and summed in fp32.
//
// MXFP8 (Miles page, section MXFP8格式背景: 32 E4M3 values per E8M0 scale).
// Each element is decoded, with its block's scale, to bf16 by
// v_cvt_scalef32_pk_bf16_fp8 (two per instruction; the converter takes only
// the exponent of its fp32 scale operand, which is exactly what an E8M0 scale
// is): an E4M3 value has at most 4 significant bits, so the decoded value is
// exact whenever it is a bf16 number, and a product of two such values is
// exact in the fp32 accumulator of v_mfma_f32_32x32x16_bf16.  gfx950's scaled
// fp8 MFMA would need no decode, but it sums each 32-block's products in a
// fixed-point window about 15 bits below the block's largest product, an
// error of up to 2^-9 sum|ab| (measured), far above the 1e-5 sum|ab| this
// GEMM promises.
//
// The fast path (k % 128 == 0) is the one-wave LDS tile kernel of gemm.hip,
// instantiated for MXFP8 (64-element stages, E8M0 scales per stage pair).
// Other shapes take the kernel below: four waves share a 256 x 256 block
// tile (each wave 128 x 128, 4 x 4 MFMA tiles) staged 128 K-elements at a
// time through LDS by register loads, with the XCD-aware tile order of
// tile_sched.h.  Lane (li, h) reads, for 32-block u of a stage, the 16-byte
// chunk 2u + h of its row (A) or column (B): K positions inside a block are
// permuted the same way for A and B, so the dot products are unchanged.
// Loads for the next stage are issued before the current stage's MFMAs and
// written to LDS after them (a mask applied right after each load would wait
// for it before the next is issued).
#include "gemm_common.h"

namespace nvfp4 {

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

// v if ok, else zeros (component-wise, so no aggregate select is formed)
__device__ __forceinline__ uint4 keep_if(bool ok, const uint4& v) {
  const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Four E8M0 codes of blocks [b, b + 4) of a scale row of nblk codes; blocks
// past the row read as 127 (2^0; their data is zero).  FULL: nblk % 4 == 0,
// one aligned dword.
template <bool FULL>
__device__ __forceinline__ uint32_t mx_scales4(const uint8_t* row, int64_t b, int64_t nblk) {
  if (FULL) return *reinterpret_cast<const uint32_t*>(row + b);
  uint32_t v = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) v |= (b + i < nblk ? (uint32_t)row[b + i] : 127u) << (8 * i);
  return v;
}

constexpr int MXL_BM = 256, MXL_BN = 256, MXL_BK = 128;

__device__ __forceinline__ int mxl_swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <bool FULL>
__global__ __launch_bounds__(256) void mxfp8_gemm_shared_kernel(MxGemmArgs p) {
  __shared__ int32_t s_prefix[SCHED_LDS_WORDS];
  __shared__ uint4 s_a[2][MXL_BM * MXL_BK / 16];
  __shared__ uint4 s_b[2][MXL_BN * MXL_BK / 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  TileRange tr;
  if (!schedule_tile<MXL_BM, MXL_BN>(p.t, lane, s_prefix, tr)) return;  // block-uniform
  const int64_t row_lo = tr.row_lo, row_hi = tr.row_hi, n0 = tr.n0;
  const uint8_t* bq = p.b_q + (int64_t)tr.g * p.n * p.k;
  const uint8_t* bsc = p.b_sc + (int64_t)tr.g * p.n * (p.k / 32);
  const int64_t nblk = p.k / 32;

  // cooperative loader: thread t moves chunks c = t + 256 i (i < 8) of each
  // operand tile: row c / 8, 16-byte column c % 8 (8 threads per 128-byte row)
  const int lcol = tid & 7;
  uint32_t lrow_a[8];
  uint32_t lmask_a = 0, lmask_b = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int64_t src = gathered_row(p.row_index, p.a_rows, row_lo + r, row_hi);
    lrow_a[i] = src >= 0 ? (uint32_t)src : 0u;
    lmask_a |= (src >= 0 ? 1u : 0u) << i;
    lmask_b |= (n0 + r < p.n ? 1u : 0u) << i;
  }
  // scale rows of this lane's fragments (wave quarter, slab i / j, row li)
  uint32_t srow_a[4];
  uint32_t smask_a = 0, smask_b = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t src = gathered_row(p.row_index, p.a_rows, row_lo + 128 * wm + 32 * i + li, row_hi);
    srow_a[i] = src >= 0 ? (uint32_t)src : 0u;
    smask_a |= (src >= 0 ? 1u : 0u) << i;
    smask_b |= (n0 + 128 * wn + 32 * i + li < p.n ? 1u : 0u) << i;
  }
  // B row of loader chunk i / scale slab i (B rows past n use row 0, masked)
  const int64_t brow0 = n0 + (tid >> 3), bsrow0 = n0 + 128 * wn + li;
#define NVFP4_MXL_GLOAD(k0, ra, rb, sa, sb)                                                    \
  do {                                                                                        \
    const bool kin = FULL || (k0) + 16 * lcol < p.k; /* chunk inside the row (k % 32 == 0) */  \
    const int64_t ko = kin ? (k0) + 16 * lcol : 0;                                            \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                           \
      const bool oka = (lmask_a >> i) & 1u, okb = (lmask_b >> i) & 1u;                        \
      const uint8_t* pa = (oka ? p.a_q + (int64_t)lrow_a[i] * p.k : p.b_q) + ko;              \
      const uint8_t* pb = (okb ? bq + (brow0 + 32 * i) * p.k : p.b_q) + ko;                   \
      ra[i] = *reinterpret_cast<const uint4*>(pa);                                            \
      rb[i] = *reinterpret_cast<const uint4*>(pb);                                            \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                           \
      const bool oka = (smask_a >> i) & 1u, okb = (smask_b >> i) & 1u;                        \
      sa[i] = mx_scales4<FULL>((oka ? p.a_sc + (int64_t)srow_a[i] * nblk : p.b_sc),           \
                               (k0) / 32, oka ? nblk : 0);                                    \
      sb[i] = mx_scales4<FULL>((okb ? bsc + (bsrow0 + 32 * i) * nblk : p.b_sc), (k0) / 32,    \
                               okb ? nblk : 0);                                               \
    }                                                                                         \
  } while (0)
#define NVFP4_MXL_LWRITE(buf, k0, ra, rb)                                              \
  do {                                                                                \
    const bool kin = FULL || (k0) + 16 * lcol < p.k;                                  \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                   \
      const int r = (tid >> 3) + 32 * i;                                              \
      const int slot = r * 8 + (lcol ^ mxl_swz(r));                                   \
      s_a[buf][slot] = keep_if(kin && ((lmask_a >> i) & 1u), ra[i]);                  \
      s_b[buf][slot] = keep_if(kin && ((lmask_b >> i) & 1u), rb[i]);                  \
    }                                                                                 \
  } while (0)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){0};

  const int64_t nstages = (p.k + MXL_BK - 1) / MXL_BK;
  uint4 ra[8], rb[8];
  uint32_t sa_cur[4], sb_cur[4], sa_nxt[4], sb_nxt[4];
  if (nstages > 0) {
    NVFP4_MXL_GLOAD(0, ra, rb, sa_cur, sb_cur);
    NVFP4_MXL_LWRITE(0, 0, ra, rb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa_cur[i] = ((smask_a >> i) & 1u) ? sa_cur[i] : 0x7F7F7F7Fu;
      sb_cur[i] = ((smask_b >> i) & 1u) ? sb_cur[i] : 0x7F7F7F7Fu;
    }
  }
  __syncthreads();
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < nstages) NVFP4_MXL_GLOAD((s + 1) * MXL_BK, ra, rb, sa_nxt, sb_nxt);
    // keep the compiler from sinking the loads' consumers (the LDS writes)
    // above the MFMAs or hoisting both K steps' fragment reads together
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // 32-block u of the stage: lane (li, h) takes 16-byte chunk 2u + h of
      // each row (its K elements all lie in block u) and the block's E8M0
      // code as the converter's scale
      uint4 qa[4], qb[4];
      float sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 128 * wm + 32 * i + li;
        qa[i] = s_a[buf][r * 8 + ((2 * u + h) ^ mxl_swz(r))];
        sa[i] = e8m0_scale((sa_cur[i] >> (8 * u)) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 128 * wn + 32 * j + li;
        qb[j] = s_b[buf][c * 8 + ((2 * u + h) ^ mxl_swz(c))];
        sb[j] = e8m0_scale((sb_cur[j] >> (8 * u)) & 0xFFu);
      }
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = mx_decode8(v ? qa[i].z : qa[i].x, v ? qa[i].w : qa[i].y, sa[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = mx_decode8(v ? qb[j].z : qb[j].x, v ? qb[j].w : qb[j].y, sb[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the stage's MFMAs are issued before the LDS writes below wait for the
    // next stage's loads (an empty asm consuming the accumulators pins them)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j])::"memory");
    if (s + 1 < nstages) {
      NVFP4_MXL_LWRITE(buf ^ 1, (s + 1) * MXL_BK, ra, rb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_cur[i] = ((smask_a >> i) & 1u) ? sa_nxt[i] : 0x7F7F7F7Fu;
        sb_cur[i] = ((smask_b >> i) & 1u) ? sb_nxt[i] : 0x7F7F7F7Fu;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int64_t row = row_lo + 128 * wm + 32 * i + 8 * (rr >> 2) + 4 * h + (rr & 3);
      if (row >= row_hi) continue;
      float* yr = p.y + row * p.n;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + 128 * wn + 32 * j + li;
        if (col < p.n) __builtin_nontemporal_store(acc[i][j][rr], yr + col);
      }
    }
  }
#undef NVFP4_MXL_GLOAD
#undef NVFP4_MXL_LWRITE
}

static void launch_mx(const MxGemmArgs& a, bool grouped, hipStream_t stream) {
  GemmArgs g{};
  g.a_q = a.a_q; g.a_sb = a.a_sc; g.a_s = nullptr; g.a_rows = a.a_rows;
  g.row_index = a.row_index; g.b_q = a.b_q; g.b_sb = a.b_sc; g.b_s = nullptr;
  g.n = a.n; g.k = a.k; g.y = a.y; g.t = a.t;
  if (launch_mxfp8_lds(g, grouped, stream)) return;
  MxGemmArgs p = a;
  const int64_t blocks = plan_tiles<MXL_BM, MXL_BN>(p.t, p.n, grouped, 1);
  if (p.k % MXL_BK == 0)
    hipLaunchKernelGGL(mxfp8_gemm_shared_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(mxfp8_gemm_shared_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       p);
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
  if (m > ((int64_t)1 << 31) || n > ((int64_t)1 << 31) || k > ((int64_t)1 << 24) ||
      !nvfp4::tile_grid_ok(m, 0, n))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(y, 16)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.e4m3_codes(a_q, m * k);
    chk.e8m0_codes(a_sc, m * (k / 32));
    chk.e4m3_codes(b_q, n * k);
    chk.e8m0_codes(b_sc, n * (k / 32));
    if ((st = chk.result())) return st;
  }
#endif
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
      k > ((int64_t)1 << 24) || !nvfp4::tile_grid_ok(m_total, groups, n))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(y, 16) || !aligned(offsets, 4) ||
      !aligned(row_index, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.e4m3_codes(a_q, a_rows * k);
    chk.e8m0_codes(a_sc, a_rows * (k / 32));
    chk.e4m3_codes(b_q, groups * n * k);
    chk.e8m0_codes(b_sc, groups * n * (k / 32));
    chk.offsets(offsets, groups);
    if ((st = chk.result())) return st;
  }
#endif
  nvfp4::MxGemmArgs p{};
  p.a_q = a_q; p.a_sc = a_sc; p.a_rows = a_rows; p.row_index = row_index;
  p.b_q = b_q; p.b_sc = b_sc; p.n = n; p.k = k; p.y = y;
  p.t.m_total = m_total; p.t.offsets = offsets; p.t.groups = (int)groups;
  nvfp4::launch_mx(p, true, (hipStream_t)stream);
  return nvfp4host::launch_status();
}
