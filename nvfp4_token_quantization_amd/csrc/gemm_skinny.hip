// gemm_skinny.hip -- the block-scaled W4A4 GEMM (dense and grouped) for few
// rows: rollout decode, where a handful of tokens, or of routed rows per
// expert, meet a whole weight (the Miles page, section 实验结果, rollout
// timing; the decode shapes are bound by the weight stream from HBM, not by
// the MFMAs).
//
// Same product and exact decode as the tiled kernels in gemm.hip:
//   Y[m, n] = S_A[m] * S_B * sum_k u_A[m, k] * u_B[n, k],  u = s_b * e2m1(q),
// every u decoded exactly to fp16, here on v_mfma_f32_16x16x32_f16.  What
// differs is how the work is split, because a 128 x 128 output tile per wave
// leaves most of the chip idle when M is 64:
//  - a workgroup owns one item: dense, up to 64 rows by 48 columns, K split
//    over up to 8 waves, each taking a contiguous run of 256-element chunks
//    (two 128-element pieces; K % 256 == 0); grouped, up to 32 rows of one
//    expert by 48 columns, K split over up to 3 waves;
//  - a chunk's operand bytes reach the wave's private LDS by DMA
//    (buffer_load ... lds, no VGPRs): four consecutive lanes read one row's
//    64-byte piece segment, so one instruction moves 16 rows x 64 bytes and
//    the vector L1 merges its lanes.  Register loads in any MFMA layout put
//    consecutive lanes on different rows; the L1 then handles every lane on
//    its own (about 62 accesses per instruction, measured), and on the
//    dense decode shape those lookups, not HBM, set the kernel time.  Rows
//    and columns that do not exist get an out-of-range buffer offset and
//    read as zeros;
//  - lane (li, g) = (lane % 16, lane / 16) then reads from LDS, for each
//    16-row slab, 16 bytes of row li: the 32 elements [32 g, 32 g + 32) of
//    the piece, so the MFMA's K slot 8 g + e of k-step (piece t, dword q) is
//    element 128 t + 32 g + 8 q + e.  A and B use the same map, so the dot
//    products are unchanged;
//  - the KS partial tiles meet in LDS; wave w sums rows w, w + KS, ... in
//    wave order (deterministic, no atomics, no workspace), scales them by
//    S_A[source row] * S_B and stores whole rows, 64 columns per instruction
//    (a one-wave item scales and stores its accumulators directly);
//  - grouped launches are persistent: four workgroups per CU walk the items
//    of the per-expert prefix of 32-row m-tiles, derived once per workgroup
//    from the device offsets.
#include "gemm_common.h"

namespace nvfp4 {

constexpr int SK_PIECE = 128;    // K elements per piece (64 bytes of a row)
constexpr int SK_NT = 2;         // pieces per chunk (one DMA round)
// A wave's stage buffer for AS 16-row A slabs and TN 16-column B slabs: code
// blocks [slab][piece] of 16 rows x 64 bytes (1 KiB, one DMA instruction
// each; slabs 0..AS-1 hold A rows, AS.. the B columns), then scales
// [slab][16 rows][8 SK_NT bytes], four slabs of one operand per DMA
// instruction (A's first, then B's).
constexpr int SK_SCALE_SLAB = 16 * 8 * SK_NT;
static_assert(SK_SCALE_SLAB * 4 == 1024, "four scale slabs per DMA instruction");
template <int AS, int TN>
constexpr int sk_code_bytes() { return (AS + TN) * SK_NT * 1024; }
template <int AS>
constexpr int sk_ascale_instr() { return (AS + 3) / 4; }
template <int TN>
constexpr int sk_bscale_instr() { return (TN + 3) / 4; }
template <int AS, int TN>
constexpr int sk_wave_bytes() {
  return sk_code_bytes<AS, TN>() + (sk_ascale_instr<AS>() + sk_bscale_instr<TN>()) * 1024;
}

struct SkinnyArgs {
  GemmArgs g;
  int ks;          // waves per workgroup (K split), <= the kernel's KSMAX
  int64_t pieces;  // K / SK_PIECE
  int nblocks;     // column blocks of 16 TN
  int bm;          // rows per item: 16 AS
  int64_t items;   // dense: m-tiles * nblocks (grouped: from the device prefix)
};

constexpr uint32_t SK_OOB = 0x80000000u;  // past every operand (operands < 2^31 bytes)

// 16-byte chunks of a 64-byte row segment sit in LDS XOR-swizzled by
// ((r >> 1) & 3): the MFMA-layout reads of 8 lanes (rows r..r+7, one chunk)
// then hit 8 different 4-bank groups.
__device__ __forceinline__ int sk_swz(int r) { return (r >> 1) & 3; }

// DMA of chunk c (K elements [256 c, 256 c + 256)) of every operand row of
// the item into the wave's stage buffer at LDS address `buf`: VS A slabs and
// TN B slabs of 16 rows x 64 bytes per piece, then 16 scale bytes per row.
template <int VS, int AS, int TN>
__device__ __forceinline__ void sk_issue(const i32x4& ra, const i32x4& ras, const i32x4& rb,
                                         const i32x4& rbs, const uint32_t (&aoff)[VS],
                                         const uint32_t (&boff)[TN],
                                         const uint32_t (&asoff)[sk_ascale_instr<AS>()],
                                         const uint32_t (&bsoff)[sk_bscale_instr<TN>()], uint32_t c,
                                         uint32_t buf) {
  constexpr int CB = sk_code_bytes<AS, TN>(), NA = sk_ascale_instr<AS>(), NB = sk_bscale_instr<TN>();
  const uint32_t kb = c * (SK_NT * SK_PIECE / 2);   // code byte of the chunk in a row
  const uint32_t kq = c * (SK_NT * SK_PIECE / 16);  // scale byte of the chunk in a row
#pragma unroll
  for (int t = 0; t < SK_NT; ++t) {
#pragma unroll
    for (int j = 0; j < TN; ++j) dma16(rb, boff[j], kb + 64u * t, buf + ((AS + j) * SK_NT + t) * 1024);
#pragma unroll
    for (int i = 0; i < VS; ++i) dma16(ra, aoff[i], kb + 64u * t, buf + (i * SK_NT + t) * 1024);
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) dma16(rbs, bsoff[u], kq, buf + CB + (NA + u) * 1024);
#pragma unroll
  for (int u = 0; u < NA; ++u) dma16(ras, asoff[u], kq, buf + CB + u * 1024);
}
template <int VS, int AS, int TN>
constexpr int sk_dma_per_chunk() {
  return SK_NT * (VS + TN) + sk_ascale_instr<AS>() + sk_bscale_instr<TN>();
}

// The MFMAs of one staged chunk (its two pieces, four k-steps each).
template <int VS, int AS, int TN>
__device__ __forceinline__ void sk_compute(const uint8_t* lds, int li, int gq, f32x4 (&acc)[VS][TN]) {
  constexpr int NT = SK_NT, CB = sk_code_bytes<AS, TN>();
  constexpr int SB = CB + sk_ascale_instr<AS>() * 1024;  // B's scale slabs
  // lane (li, g) reads chunk g of row li; its scale dword g / 2 of the
  // piece's two holds blocks 4 (g / 2) .. + 3, of which it uses bytes
  // 2 (g & 1) + q / 2
  const int rchunk = (gq ^ sk_swz(li)) * 16;
  const int sbyte = 2 * (gq & 1);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint4 qa[VS], qb[TN];
    uint32_t sa[VS], sb[TN];
#pragma unroll
    for (int i = 0; i < VS; ++i) {
      qa[i] = *reinterpret_cast<const uint4*>(lds + (i * NT + t) * 1024 + li * 64 + rchunk);
      sa[i] = *reinterpret_cast<const uint32_t*>(lds + CB + i * SK_SCALE_SLAB + li * 16 + 8 * t +
                                                 4 * (gq >> 1));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      qb[j] = *reinterpret_cast<const uint4*>(lds + ((AS + j) * NT + t) * 1024 + li * 64 + rchunk);
      sb[j] = *reinterpret_cast<const uint32_t*>(lds + SB + j * SK_SCALE_SLAB + li * 16 + 8 * t +
                                                 4 * (gq >> 1));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int blk = sbyte + (q >> 1);
      f16x8 fa[VS], fb[TN];
#pragma unroll
      for (int i = 0; i < VS; ++i) fa[i] = decode8(pick(qa[i], q), scale_pair(sa[i], blk));
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = decode8(pick(qb[j], q), scale_pair(sb[j], blk));
#pragma unroll
      for (int i = 0; i < VS; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      // keep each k-step's decode next to its MFMAs (hoisting the whole
      // chunk's decode would need a register per decoded operand)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One item: rows [row_lo, row_hi) (VS 16-row slabs) by columns [n0, n0 +
// 16 TN) of expert g, K split over the workgroup's p.ks <= KSMAX waves,
// NBUF stage buffers per wave (2: the DMA of chunk c + 1 overlaps the MFMAs
// of chunk c).  Called by every wave of the workgroup.  Index arithmetic is
// 32-bit (rows, columns and chunks all fit): 64-bit divisions here cost
// more than a microsecond before the first DMA.
template <int VS, int AS, int TN, int NBUF, int KSMAX>
__device__ __forceinline__ void skinny_item(const SkinnyArgs& p, int wave, int lane, int row_lo,
                                            int row_hi, int n0, int g, uint8_t* s_stage) {
  constexpr int WB = sk_wave_bytes<AS, TN>();
  constexpr int NA = sk_ascale_instr<AS>(), NB = sk_bscale_instr<TN>();
  const GemmArgs& a = p.g;
  const int li = lane & 15, gq = lane >> 4;
  const int n = (int)a.n;
  const uint32_t rowb = (uint32_t)(a.k / 2), rows_s = (uint32_t)(a.k / 16);
  const i32x4 ra = make_rsrc(a.a_q, a.a_rows * rowb);
  const i32x4 ras = make_rsrc(a.a_sb, a.a_rows * rows_s);
  const i32x4 rb = make_rsrc(a.b_q + (int64_t)g * a.n * rowb, a.n * rowb);
  const i32x4 rbs = make_rsrc(a.b_sb + (int64_t)g * a.n * rows_s, a.n * rows_s);
  // DMA lanes: codes of row lane / 4 of each slab, global chunk (lane & 3) ^
  // swz into LDS chunk lane & 3; scales of row lane & 15 of slab 4 u +
  // lane / 16 of scale instruction u
  const int cr = lane >> 2, sl = lane >> 4, srow = lane & 15;
  const uint32_t cchunk = (uint32_t)(((lane & 3) ^ sk_swz(cr)) * 16);
  uint32_t boff[TN], bsoff[NB];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + 16 * j + cr;
    boff[j] = col < n ? (uint32_t)col * rowb + cchunk : SK_OOB;
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int col = n0 + 16 * (4 * u + sl) + srow;
    bsoff[u] = (4 * u + sl < TN && col < n) ? (uint32_t)col * rows_s : SK_OOB;
  }
  // the source A row of output row row_lo + lane (a load only with a row
  // index); lanes past the item's 16 AS rows hold -1
  const int32_t src = lane >= 16 * AS ? -1
                      : a.row_index ? (int32_t)gathered_row(a.row_index, a.a_rows, row_lo + lane, row_hi)
                                    : (row_lo + lane < row_hi ? row_lo + lane : -1);
  uint32_t aoff[VS], asoff[NA];
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    const int32_t r = __shfl(src, 16 * i + cr, 64);
    aoff[i] = r >= 0 ? (uint32_t)r * rowb + cchunk : SK_OOB;
  }
#pragma unroll
  for (int u = 0; u < NA; ++u) {
    const int32_t r = __shfl(src, (16 * (4 * u + sl) + srow) & 63, 64);
    asoff[u] = (4 * u + sl < VS && r >= 0) ? (uint32_t)r * rows_s : SK_OOB;
  }
  const int wu = __builtin_amdgcn_readfirstlane(wave);  // the DMA's scalar operands are built from it
  const uint32_t wbase = (uint32_t)(uintptr_t)s_stage + (uint32_t)wu * (NBUF * WB);
  const uint8_t* lds = s_stage + wave * (NBUF * WB);

  f32x4 acc[VS][TN];
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // this wave's chunks: a contiguous run, the first (chunks % ks) waves one more
  const uint32_t chunks = (uint32_t)(p.pieces / SK_NT), ks = (uint32_t)p.ks;
  const uint32_t per = chunks / ks, extra = chunks % ks;
  const uint32_t cbeg = (uint32_t)wu * per + min((uint32_t)wu, extra);
  const uint32_t cend = cbeg + per + ((uint32_t)wu < extra ? 1u : 0u);
  constexpr int ND = sk_dma_per_chunk<VS, AS, TN>();
  if (cbeg < cend) sk_issue<VS, AS, TN>(ra, ras, rb, rbs, aoff, boff, asoff, bsoff, cbeg, wbase);
  for (uint32_t c = cbeg; c < cend; ++c) {
    const int b = NBUF == 2 ? (int)((c - cbeg) & 1u) : 0;
    if (NBUF == 2 && c + 1 < cend) {
      // chunk c + 1 into the other buffer (its last reads were waited for
      // at the end of chunk c - 1), then wait for chunk c only
      sk_issue<VS, AS, TN>(ra, ras, rb, rbs, aoff, boff, asoff, bsoff, c + 1, wbase + (b ^ 1) * WB);
      wait_vmcnt<ND>();
    } else {
      wait_vmcnt<0>();
    }
    sk_compute<VS, AS, TN>(lds + b * WB, li, gq, acc);
    wait_lgkmcnt0();  // the chunk's reads have landed before its buffer is refilled
    if (NBUF == 1 && c + 1 < cend)
      sk_issue<VS, AS, TN>(ra, ras, rb, rbs, aoff, boff, asoff, bsoff, c + 1, wbase);
  }

  const float rs = (src >= 0 ? a.a_s[src] : 0.0f) * a.b_s[g];
  const int rows = row_hi - row_lo;
  if (KSMAX == 1) {
    // one wave: each lane stores its own entries, row 16 i + 4 g + w (scale
    // from the lane that holds that row's source) by column 16 j + li
#pragma unroll
    for (int i = 0; i < VS; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int r = 16 * i + 4 * gq + w;
        const float sr = __shfl(rs, r, 64);
        if (r < rows) {
          float* yr = a.y + (int64_t)(row_lo + r) * n;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + 16 * j + li;
            if (col < n) __builtin_nontemporal_store(acc[i][j][w] * sr, yr + col);
          }
        }
      }
    return;
  }
  // Every wave puts its partial tile in LDS (entry-major, lane-minor, over
  // the staging buffers, so all waves must be done with those first), and
  // wave 0 the epilogue scale of each row, S_A of its source row times S_B,
  // after them; then wave w sums, in wave order, rows w, w + ks, ... and
  // stores them.  Lane (li, g), accumulator entry w holds row 16 i + 4 g + w,
  // column 16 j + li.
  constexpr int NE = VS * TN * 4;
  float* s_red = reinterpret_cast<float*>(s_stage);
  float* s_rs = s_red + KSMAX * AS * TN * 4 * 64;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) s_red[(wave * NE + (i * TN + j) * 4 + w) * 64 + lane] = acc[i][j][w];
  if (wave == 0 && lane < 16 * AS) s_rs[lane] = rs;
  __syncthreads();
#pragma unroll
  for (int c0 = 0; c0 < 16 * TN; c0 += 64) {
    const int cc = c0 + lane, col = n0 + cc;
    if (cc < 16 * TN && col < n) {
      const int cj = cc >> 4, cl = cc & 15;
      for (int r = wave; r < rows; r += p.ks) {
        // entry (16 i + 4 g + w, 16 j + l) sits in lane l + 16 g, entry
        // (i TN + j) 4 + w; all ks partials are read before the sum
        const int e = ((r >> 4) * TN + cj) * 4 + (r & 3);
        const int ln = cl + 16 * ((r >> 2) & 3);
        float part[KSMAX];
#pragma unroll
        for (int k = 0; k < KSMAX; ++k) part[k] = k < p.ks ? s_red[(k * NE + e) * 64 + ln] : 0.0f;
        float v = part[0];
#pragma unroll
        for (int k = 1; k < KSMAX; ++k) v += part[k];
        __builtin_nontemporal_store(v * s_rs[r], a.y + (int64_t)(row_lo + r) * n + col);
      }
    }
  }
}

// AS: 16-row A slabs per item (rows per item 16 AS); TN: 16-column B slabs
// per item; KSMAX: most waves per workgroup; NBUF: stage buffers per wave.
// A grouped launch (one wave per workgroup; with one stage buffer at most
// 256 VGPRs, so that two share a SIMD) keeps the expert prefix in dynamic
// LDS of 4 (3 G + 1) bytes.
template <int AS, int TN, int KSMAX, int NBUF, bool GROUPED>
__global__ __launch_bounds__(64 * KSMAX) __attribute__((amdgpu_waves_per_eu(GROUPED && NBUF == 1 ? 2 : 1)))
void gemm_skinny_kernel(SkinnyArgs p) {
  constexpr int BM = 16 * AS;
  extern __shared__ int32_t s_dyn[];
  // staging buffers; after the K loop the partial tiles, then the row scales
  constexpr int STAGE = KSMAX * NBUF * sk_wave_bytes<AS, TN>();
  constexpr int RED = KSMAX > 1 ? (KSMAX * AS * TN * 4 * 64 + BM) * 4 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[STAGE > RED ? STAGE : RED];
  const GemmArgs& a = p.g;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.t.groups;
  const int m_total = (int)a.t.m_total;
  int32_t* s_prefix = s_dyn;
  int32_t* s_lo = s_dyn + G + 1;
  int32_t* s_hi = s_lo + G;
  int items = (int)p.items;
  if (GROUPED) {
    if (wave == 0) expert_tile_prefix<BM>(a.t.offsets, G, a.t.m_total, lane, s_prefix, s_lo, s_hi);
    if (KSMAX > 1) __syncthreads();
    else wave_lds_sync();
    items = s_prefix[G] * p.nblocks;
  }
  for (int it = blockIdx.x; it < items; it += gridDim.x) {  // workgroup-uniform
    const int mt = it / p.nblocks;
    const int n0 = (it - mt * p.nblocks) * 16 * TN;
    int g = 0, row_lo, row_hi;
    if (GROUPED) {
      g = find_expert(s_prefix, G, mt, lane);
      row_lo = s_lo[g] + (mt - s_prefix[g]) * BM;
      row_hi = min(s_hi[g], row_lo + BM);
    } else {
      row_lo = mt * BM;
      row_hi = min(m_total, row_lo + BM);
    }
    const int vs = (row_hi - row_lo + 15) >> 4;  // 16-row slabs that hold rows
    if (AS == 1 || vs <= 1) skinny_item<1, AS, TN, NBUF, KSMAX>(p, wave, lane, row_lo, row_hi, n0, g, s_stage);
    else if (AS == 2 || vs == 2) skinny_item<(AS >= 2 ? 2 : 1), AS, TN, NBUF, KSMAX>(p, wave, lane, row_lo, row_hi, n0, g, s_stage);
    else if (AS == 3 || vs == 3) skinny_item<(AS >= 3 ? 3 : 1), AS, TN, NBUF, KSMAX>(p, wave, lane, row_lo, row_hi, n0, g, s_stage);
    else skinny_item<AS, AS, TN, NBUF, KSMAX>(p, wave, lane, row_lo, row_hi, n0, g, s_stage);
    if (KSMAX > 1) __syncthreads();  // the LDS is free for the next item
  }
}

bool launch_gemm_skinny(const GemmArgs& a, bool grouped, hipStream_t stream) {
  const int64_t K = a.k;
  // whole chunks only: every DMA then stays inside its row
  if (K <= 0 || K % (SK_NT * SK_PIECE) != 0 || a.a_rows <= 0) return false;
  // few rows: a dense M of at most 64, or at most 16 routed rows per expert
  // on average (the host never reads the offsets)
  if (!grouped && a.t.m_total > 64) return false;
  if (grouped && a.t.m_total > 16 * (int64_t)a.t.groups) return false;
  const int64_t lim = (int64_t)1 << 31;  // 32-bit buffer offsets with room for SK_OOB
  if (a.a_rows * (K / 2) >= lim || a.n * (K / 2) >= lim) return false;
  SkinnyArgs p;
  p.g = a;
  p.pieces = K / SK_PIECE;
  const int cus = nvfp4host::num_cus();
  int64_t grid;
  size_t dyn = 0;
  void (*k)(SkinnyArgs);
  if (!grouped) {
    // one workgroup per item of 64 rows x 48 columns (N = 9728: 203 items,
    // one round on 256 CUs), K split over up to 8 waves (one or two chunks
    // each at K = 2560; measured 12.1 us against 12.8 with 10 waves, 12.4
    // with 7, 13.3 with 9) and the partial tiles summed in LDS
    p.bm = 64;
    p.nblocks = (int)((a.n + 47) / 48);
    p.items = p.nblocks;
    p.ks = (int)min((int64_t)8, p.pieces / SK_NT);
    k = gemm_skinny_kernel<4, 3, 8, 1, false>;
    grid = p.items;
  } else {
    // items of up to 32 rows of one expert (decode experts mostly hold at
    // most 16, rarely more than 32) x 48 columns, K split over three waves
    // with one stage buffer each; four workgroups per CU.  Measured on the
    // rollout-decode shapes against one-wave items of 128 columns with two
    // buffers (three per CU) and other splits: the per-wave decode, not the
    // weight stream, bounds a one-wave item, so the K split wins.
    p.bm = 32;
    p.nblocks = (int)((a.n + 47) / 48);
    p.items = (a.t.m_total / 32 + a.t.groups) * p.nblocks;  // a bound; exact on the device
    p.ks = (int)min((int64_t)3, p.pieces / SK_NT);
    k = gemm_skinny_kernel<2, 3, 3, 1, true>;
    dyn = (size_t)(3 * a.t.groups + 1) * 4;
    // resident workgroups per CU (LDS: 160 KiB per CU)
    const int64_t wg_lds = 3 * sk_wave_bytes<2, 3>() + (int64_t)dyn;
    grid = min(p.items, (int64_t)cus * min((int64_t)4, (int64_t)163840 / wg_lds));
  }
  if (grid <= 0 || p.items >= ((int64_t)1 << 31)) return false;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * p.ks), dyn, stream, p);
  return true;
}

}  // namespace nvfp4
