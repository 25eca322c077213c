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
// Tiling: one wave per block (one per SIMD), the block tile is the wave's
// 4 x 4 tiles of v_mfma_f32_32x32x16_f16 with 256 fp32 accumulators.  A K
// stage is 128 elements; lane (li, h) holds, for each 32-row slab of A and B,
// the 32 code bytes [32h, 32h + 32) of the row's 64 and the dword of the 4
// block scales that cover them, so lane half h feeds the K elements
// [64h, 64h + 64) of every stage to the MFMAs of both operands: a
// permutation of K that is the same for A and B, so the dot products are
// unchanged.  Two ways to get the operands there:
//   gemm_lds_kernel (k % 256 == 0): global -> private LDS buffers by DMA with
//     whole row segments per instruction, then ds_reads into that layout;
//   gemm_rd_kernel (other k): each lane loads its own fragments straight into
//     a register double buffer.
//
// Tile order: blocks are dealt round-robin to the 8 XCDs; the grid is split
// into 8 regions (one per XCD, along M for grouped GEMMs) so each XCD's L2
// serves one region.  Grouped GEMMs derive the per-expert m-tile prefix from
// the device offsets in every block, and ragged expert tiles run only their
// non-empty 32-row slabs.
#include <type_traits>

#include "gemm_common.h"
#include "swiglu_core.h"

namespace nvfp4 {

constexpr int BK = 128;          // K elements per stage

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

__device__ __forceinline__ uint4 load16_codes(const uint8_t* row, int64_t off, int64_t rowb,
                                              bool fast) {
  if (fast) return *reinterpret_cast<const uint4*>(row + off);
  uint2 lo = load8_masked(row, off, rowb), hi = load8_masked(row, off + 8, rowb);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}


// ---------------------------------------------------------------------------
// Register-direct variant: one wave per block, block tile = wave tile =
// (32 TM) x (32 TN).  Each lane loads its own MFMA fragments straight from
// global memory (L2) into a register double buffer one K stage ahead: lane
// (li, h) reads, for every 32-row slab, 32 code bytes [32h, 32h + 32) of the
// stage's 64 and the dword of 4 block scales covering them.  No LDS staging
// and no barriers in the K loop; LDS only holds the per-row epilogue scales.
template <int TM, int TN>
struct RegStage {
  uint4 a[TM][2];
  uint4 b[TN][2];
  uint32_t as[TM];
  uint32_t bs[TN];
};

__device__ __forceinline__ uint32_t load4_bytes(const uint8_t* row, int64_t off, int64_t valid) {
  uint32_t v = 0u;
  for (int i = 0; i < 4; ++i)
    if (off + i < valid) v |= (uint32_t)row[off + i] << (8 * i);
  return v;
}

template <int TM, int TN, int VS, bool FAST>
__device__ __forceinline__ void rd_load(const GemmArgs& p, const uint8_t* const* arow,
                                        const uint8_t* const* asrow, const uint8_t* const* brow,
                                        const uint8_t* const* bsrow, int h, int64_t k0,
                                        RegStage<TM, TN>& r) {
  const int64_t rowb = p.k / 2, rows_s = p.k / 16;
  const int64_t off = k0 / 2 + 32 * h;
  const int64_t soff = k0 / 16 + 4 * h;
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    if (!arow[i]) {
      r.a[i][0] = r.a[i][1] = make_uint4(0, 0, 0, 0);
      r.as[i] = 0;
    } else if (FAST) {
      const uint4* q = reinterpret_cast<const uint4*>(arow[i] + off);
      r.a[i][0] = q[0];
      r.a[i][1] = q[1];
      r.as[i] = *reinterpret_cast<const uint32_t*>(asrow[i] + soff);
    } else {
      r.a[i][0] = load16_codes(arow[i], off, rowb, false);
      r.a[i][1] = load16_codes(arow[i], off + 16, rowb, false);
      r.as[i] = load4_bytes(asrow[i], soff, rows_s);
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (!brow[j]) {
      r.b[j][0] = r.b[j][1] = make_uint4(0, 0, 0, 0);
      r.bs[j] = 0;
    } else if (FAST) {
      const uint4* q = reinterpret_cast<const uint4*>(brow[j] + off);
      r.b[j][0] = q[0];
      r.b[j][1] = q[1];
      r.bs[j] = *reinterpret_cast<const uint32_t*>(bsrow[j] + soff);
    } else {
      r.b[j][0] = load16_codes(brow[j], off, rowb, false);
      r.b[j][1] = load16_codes(brow[j], off + 16, rowb, false);
      r.bs[j] = load4_bytes(bsrow[j], soff, rows_s);
    }
  }
}

template <int TM, int TN, int VS>
__device__ __forceinline__ void rd_compute(const RegStage<TM, TN>& r, f32x16 (&acc)[TM][TN]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    f16x8 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < VS; ++i) fa[i] = decode8(pick(r.a[i][t >> 2], t), scale_pair(r.as[i], t >> 1));
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = decode8(pick(r.b[j][t >> 2], t), scale_pair(r.bs[j], t >> 1));
#pragma unroll
    for (int i = 0; i < VS; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }
}

template <int TM, int TN, int VS, bool FAST>
__device__ __forceinline__ void rd_kloop(const GemmArgs& p, const uint8_t* const* arow,
                                         const uint8_t* const* asrow, const uint8_t* const* brow,
                                         const uint8_t* const* bsrow, int h,
                                         f32x16 (&acc)[TM][TN]) {
  const int64_t nstages = (p.k + BK - 1) / BK;
  RegStage<TM, TN> r0, r1;
  if (nstages > 0) rd_load<TM, TN, VS, FAST>(p, arow, asrow, brow, bsrow, h, 0, r0);
  // two stages per iteration so the double buffer needs no register moves
  int64_t s = 0;
  for (; s + 1 < nstages; s += 2) {
    rd_load<TM, TN, VS, FAST>(p, arow, asrow, brow, bsrow, h, (s + 1) * BK, r1);
    rd_compute<TM, TN, VS>(r0, acc);
    if (s + 2 < nstages) rd_load<TM, TN, VS, FAST>(p, arow, asrow, brow, bsrow, h, (s + 2) * BK, r0);
    rd_compute<TM, TN, VS>(r1, acc);
  }
  if (s < nstages) rd_compute<TM, TN, VS>(r0, acc);
}

// Accumulate the tile over K with VS valid A slabs, then scale and store
// (streaming stores: Y is written once and not read back by this kernel).
template <int TM, int TN, int VS, bool FAST>
__device__ __forceinline__ void rd_body(const GemmArgs& p, const uint8_t* const* arow,
                                        const uint8_t* const* asrow, const uint8_t* const* brow,
                                        const uint8_t* const* bsrow, int h, int li, int64_t row_lo,
                                        int64_t row_hi, int64_t n0, const float* s_rowscale) {
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){0};
  rd_kloop<TM, TN, VS, FAST>(p, arow, asrow, brow, bsrow, h, acc);
  __syncthreads();  // s_rowscale (written by this wave) is visible
#pragma unroll
  for (int i = 0; i < VS; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lrow = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t row = row_lo + lrow;
      if (row >= row_hi) continue;
      const float sc = s_rowscale[lrow];
      float* yr = p.y + row * p.n;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + 32 * j + li;
        if (col < p.n) __builtin_nontemporal_store(acc[i][j][r] * sc, yr + col);
      }
    }
  }
}

template <int TM, int TN, bool FAST>
__global__ __launch_bounds__(64) void gemm_rd_kernel(GemmArgs p) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  __shared__ int32_t s_prefix[SCHED_LDS_WORDS];
  __shared__ float s_rowscale[BM];

  const int lane = threadIdx.x;
  const int h = lane >> 5, li = lane & 31;

  TileRange tr;
  if (!schedule_tile<BM, BN>(p.t, lane, s_prefix, tr)) return;  // block-uniform
  const int64_t row_lo = tr.row_lo, row_hi = tr.row_hi, n0 = tr.n0;
  const int g = tr.g;
  const uint8_t* bq_base = p.b_q + (int64_t)g * p.n * (p.k / 2);
  const uint8_t* bsb_base = p.b_sb + (int64_t)g * p.n * (p.k / 16);

  // Source A rows of the tile's output rows: lane l looks up rows l and 64 + l
  // (independent loads), other lanes' rows come by shuffle (TM <= 4).
  static_assert(BM <= 128, "two rows per lane");
  const int32_t src0 = (int32_t)gathered_row(p.row_index, p.a_rows, row_lo + lane, row_hi);
  const int32_t src1 = BM > 64 ? (int32_t)gathered_row(p.row_index, p.a_rows, row_lo + 64 + lane, row_hi)
                               : -1;

  const uint8_t* arow[TM];
  const uint8_t* asrow[TM];
  const uint8_t* brow[TN];
  const uint8_t* bsrow[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t r = __shfl(i >= 2 ? src1 : src0, (32 * i + li) & 63, 64);
    arow[i] = r >= 0 ? p.a_q + r * (p.k / 2) : nullptr;
    asrow[i] = r >= 0 ? p.a_sb + r * (p.k / 16) : nullptr;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t c = n0 + 32 * j + li;
    brow[j] = c < p.n ? bq_base + c * (p.k / 2) : nullptr;
    bsrow[j] = c < p.n ? bsb_base + c * (p.k / 16) : nullptr;
  }
  {
    const float sbw = p.b_s[g];
    if (lane < BM) s_rowscale[lane] = (src0 >= 0 ? p.a_s[src0] : 0.0f) * sbw;
    if (BM > 64) s_rowscale[64 + lane] = (src1 >= 0 ? p.a_s[src1] : 0.0f) * sbw;
  }

  // K loop and epilogue over the valid 32-row slabs only (ragged expert
  // tiles skip the loads, decodes and MFMAs of empty slabs)
  const int vslabs = (int)min((int64_t)TM, (row_hi - row_lo + 31) / 32);
  static_assert(TM == 4, "slab dispatch is written for TM == 4");
  switch (vslabs) {
    case 4: rd_body<TM, TN, 4, FAST>(p, arow, asrow, brow, bsrow, h, li, row_lo, row_hi, n0, s_rowscale); break;
    case 3: rd_body<TM, TN, 3, FAST>(p, arow, asrow, brow, bsrow, h, li, row_lo, row_hi, n0, s_rowscale); break;
    case 2: rd_body<TM, TN, 2, FAST>(p, arow, asrow, brow, bsrow, h, li, row_lo, row_hi, n0, s_rowscale); break;
    default: rd_body<TM, TN, 1, FAST>(p, arow, asrow, brow, bsrow, h, li, row_lo, row_hi, n0, s_rowscale); break;
  }
}

// ---------------------------------------------------------------------------
// LDS-staged variant (k % 256 == 0, 16-byte aligned codes, operands under
// 2 GiB).  Same wave tile, MFMA layout and K permutation as the
// register-direct kernel, but every operand byte reaches the wave through a
// buffer_load ... lds (global -> LDS, no VGPRs) whose lanes read whole 64-byte
// row segments: four consecutive lanes cover one row's stage, so a 16-row
// instruction touches 16 segments where the register layout touched 64
// lane-sized pieces, which the vector L1 serves one by one.  Each wave owns
// two private LDS stage buffers (no sharing, no barriers); the DMA of stage
// s + 2 is issued while stage s is consumed, and half-stages move from LDS to
// registers one half ahead of the MFMAs.
//
// The DMA is written as inline asm: the compiler's wait insertion cannot tell
// the two stage buffers apart and would drain every DMA in flight before each
// ds_read.  The asm blocks clobber memory, and the waits are explicit:
// vmcnt before a stage is read, lgkmcnt before its buffer is refilled.
//
// LDS per wave (40 KiB, so four one-wave blocks fill a CU's 160 KiB):
//   two code stage buffers of 8 slabs (4 of A, 4 of B) x 32 rows x 64 bytes;
//     code row r keeps its four 16-byte chunks XOR-swizzled by
//     ((r >> 2) + (r & 2)) & 3, so the ds_read_b128s of any 8 (and any 16)
//     consecutive rows of an aligned group hit different 16-byte bank groups;
//   two scale buffers, each holding a PAIR of stages: 8 slabs x 32 rows x 16
//     bytes (stage 2p's 8 scale bytes, then stage 2p + 1's), loaded 16 bytes
//     per lane, so a scale DMA moves 16 bytes per row touched instead of 4.
// The epilogue's per-row scales reuse the first code buffer after the K loop,
// and the expert tile prefix (read before the K loop) the second.
constexpr int LDS_SLAB_CODES = 32 * 64;
constexpr int LDS_CODES = 8 * LDS_SLAB_CODES;   // one code stage buffer
constexpr int LDS_SCALES_AT = 2 * LDS_CODES;
// scale bytes per row and stage pair: NVFP4 2 x 8 (16-element blocks of a
// 128-element stage), MXFP8 2 x 2 (32-element blocks of a 64-element stage)
template <bool MX> constexpr int lds_slab_scales() { return 32 * (MX ? 4 : 16); }
template <bool MX> constexpr int lds_scales() { return 8 * lds_slab_scales<MX>(); }
template <bool MX> constexpr int lds_wave() { return 2 * LDS_CODES + 2 * lds_scales<MX>(); }
// K elements per stage (64 bytes of every row)
template <bool MX> constexpr int lds_bk() { return MX ? 64 : 128; }
constexpr int LDS_WAVE = lds_wave<false>();
static_assert(LDS_WAVE * 4 <= 160 * 1024, "four waves per CU");

__device__ __forceinline__ int lds_swz(int r) { return ((r >> 2) + (r & 2)) & 3; }

// Streaming 4-byte store to rsrc[voff] (dropped when voff is out of range).
__device__ __forceinline__ void store_nt(__amdgpu_buffer_rsrc_t rsrc, float v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc, voff, 0, 2);
}

struct LdsOperands {
  i32x4 aq, as, bq, bs;
  uint32_t aoff[4][2], asoff[2], boff[4][2], bsoff[2];
  uint32_t avalid, bvalid;  // bit i: this lane's MFMA row / column of slab i exists
};

// DMA of K stage `st`'s codes (64 bytes of each row) into the code buffer at
// LDS address `buf`: VS slabs of A, all four of B; 2 VS + 8 instructions.
template <int VS>
__device__ __forceinline__ void lds_issue_codes(const LdsOperands& o, uint32_t buf, uint32_t st) {
  const uint32_t sc = 64u * st;
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    dma16(o.aq, o.aoff[i][0], sc, buf + i * LDS_SLAB_CODES);
    dma16(o.aq, o.aoff[i][1], sc, buf + i * LDS_SLAB_CODES + 1024);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dma16(o.bq, o.boff[j][0], sc, buf + (4 + j) * LDS_SLAB_CODES);
    dma16(o.bq, o.boff[j][1], sc, buf + (4 + j) * LDS_SLAB_CODES + 1024);
  }
}

// DMA of the scales of stages st and st + 1 (st even) into the scale pair
// buffer at `buf`: one instruction per two slabs (lanes 0-31 the first slab's
// rows, 32-63 the second's), four instructions of 16 (NVFP4) or 4 (MXFP8)
// bytes per lane.
template <bool MX>
__device__ __forceinline__ void lds_issue_scales(const LdsOperands& o, uint32_t buf, uint32_t st) {
  constexpr int SL = lds_slab_scales<MX>();
  if (MX) {
    const uint32_t ss = 2u * st;
    dma4(o.as, o.asoff[0], ss, buf);
    dma4(o.as, o.asoff[1], ss, buf + 2 * SL);
    dma4(o.bs, o.bsoff[0], ss, buf + 4 * SL);
    dma4(o.bs, o.bsoff[1], ss, buf + 6 * SL);
  } else {
    const uint32_t ss = 8u * st;
    dma16(o.as, o.asoff[0], ss, buf);
    dma16(o.as, o.asoff[1], ss, buf + 2 * SL);
    dma16(o.bs, o.bsoff[0], ss, buf + 4 * SL);
    dma16(o.bs, o.bsoff[1], ss, buf + 6 * SL);
  }
}

// Half a stage in the MFMA register layout: lane (li, h) holds 16-byte chunk
// 2h + part of row li and a dword of block scales.  NVFP4: K elements
// [64h + 32 part, +32), and the four block scales of its 64 elements.
// MXFP8: K elements [32h + 16 part, +16) of the stage, all in the stage's
// 32-block h, and the row's scale dword of the stage pair (byte 2 odd + h is
// this lane's).
struct RegHalf {
  uint4 a[4], b[4];
  uint32_t as[4], bs[4];
};

// ds_reads of half `part` of the stage whose codes are at `buf` and whose
// scales are the `odd` half of the pair buffer `sbuf`.  Rows that do not
// exist must decode to zeros whatever their LDS bytes hold: NVFP4 gives them
// a zero scale; MXFP8 (whose converter reads a zero scale as 2^-127) zero
// codes and the scale 2^0.  Columns past n are never stored.
template <int VS, bool MX>
__device__ __forceinline__ void lds_read(const LdsOperands& o, const uint8_t* buf,
                                         const uint8_t* sbuf, int odd, int li, int h, int part,
                                         RegHalf& r) {
  constexpr int SL = lds_slab_scales<MX>();
  const int c = ((2 * h + part) ^ lds_swz(li)) * 16;
  const uint8_t* sc = MX ? sbuf + li * 4 : sbuf + li * 16 + 8 * odd + 4 * h;
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    const uint4 q = *reinterpret_cast<const uint4*>(buf + i * LDS_SLAB_CODES + li * 64 + c);
    const uint32_t sv = *reinterpret_cast<const uint32_t*>(sc + i * SL);
    const bool ok = (o.avalid >> i) & 1u;
    if (MX) {
      const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
      r.a[i] = make_uint4(q.x & m, q.y & m, q.z & m, q.w & m);
      r.as[i] = ok ? sv : 0x7F7F7F7Fu;
    } else {
      r.a[i] = q;
      r.as[i] = ok ? sv : 0u;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.b[j] = *reinterpret_cast<const uint4*>(buf + (4 + j) * LDS_SLAB_CODES + li * 64 + c);
    const uint32_t sv = *reinterpret_cast<const uint32_t*>(sc + (4 + j) * SL);
    r.bs[j] = MX ? sv : (((o.bvalid >> j) & 1u) ? sv : 0u);
  }
}

template <bool MX>
using lds_op_t = typename std::conditional<MX, bf16x8, f16x8>::type;

// Decode of one k-step.  NVFP4: dword t of each 16-byte chunk with block
// scale byte blk.  MXFP8: dwords 2t and 2t + 1 with the E8M0 code in byte
// blk of the scale dword.
template <int VS, bool MX>
__device__ __forceinline__ void decode_step(const RegHalf& r, int t, int blk,
                                            lds_op_t<MX> (&fa)[4], lds_op_t<MX> (&fb)[4]) {
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < VS; ++i)
      fa[i] = mx_decode8(t ? r.a[i].z : r.a[i].x, t ? r.a[i].w : r.a[i].y,
                         e8m0_scale((r.as[i] >> (8 * blk)) & 0xFFu));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j] = mx_decode8(t ? r.b[j].z : r.b[j].x, t ? r.b[j].w : r.b[j].y,
                         e8m0_scale((r.bs[j] >> (8 * blk)) & 0xFFu));
  } else {
#pragma unroll
    for (int i = 0; i < VS; ++i) fa[i] = decode8(pick(r.a[i], t), scale_pair(r.as[i], blk));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = decode8(pick(r.b[j], t), scale_pair(r.bs[j], blk));
  }
}

// One k-step: the MFMAs of the decoded operands (fa, fb) while the next
// k-step (nt, scale byte nblk of `nr`) is decoded, interleaved one MFMA to a
// few VALU instructions so the decode issues in the MFMAs' shadow.
template <int VS, bool MX>
__device__ __forceinline__ void kstep(f32x16 (&acc)[4][4], lds_op_t<MX> (&fa)[4],
                                      lds_op_t<MX> (&fb)[4], const RegHalf& nr, int nt, int nblk) {
  lds_op_t<MX> na[4], nb[4];
  decode_step<VS, MX>(nr, nt, nblk, na, nb);
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MX)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  // VALU per operand decode: 9 (NVFP4: 4 converts, 4 scale multiplies, the
  // scale pair), 6 (MXFP8: 4 converts, the scale's shift and mask)
  constexpr int NM = 4 * VS, NV = ((VS + 4) * (MX ? 6 : 9) + NM - 1) / NM;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // then up to NV VALU
  }
#pragma unroll
  for (int i = 0; i < VS; ++i) fa[i] = na[i];
#pragma unroll
  for (int j = 0; j < 4; ++j) fb[j] = nb[j];
}

template <int VS, bool MX, bool SW = false>
__device__ __forceinline__ void lds_body(const GemmArgs& p, const LdsOperands& o, uint8_t* lds,
                                         int h, int li, int lane, int64_t row_lo, int64_t row_hi,
                                         int64_t n0, float rs0, float rs1) {
  constexpr int NC = 2 * VS + 8;  // code DMA instructions per stage
  constexpr int NS = 4;           // scale DMA instructions per stage pair
  constexpr int SCALES = lds_scales<MX>();
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < VS; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){0};
  const uint32_t lbase = (uint32_t)(uintptr_t)lds;  // LDS address (low 32 bits)
  const int nst = (int)(p.k / lds_bk<MX>());         // even and >= 2 on this path
  RegHalf r0, r1;
  lds_op_t<MX> fa[4], fb[4];
  // stage s: codes in code buffer s & 1, scales in pair buffer (s >> 1) & 1.
  // In flight at most: codes of two stages and scales of two pairs.
  lds_issue_scales<MX>(o, lbase + LDS_SCALES_AT, 0);
  lds_issue_codes<VS>(o, lbase, 0);
  lds_issue_codes<VS>(o, lbase + LDS_CODES, 1);
  if (nst > 2) {
    lds_issue_scales<MX>(o, lbase + LDS_SCALES_AT + SCALES, 2);
    wait_vmcnt<NC + NS>();  // stage 0's codes and scales are in LDS
  } else {
    wait_vmcnt<NC>();
  }
  lds_read<VS, MX>(o, lds, lds + LDS_SCALES_AT, 0, li, h, 0, r0);
  decode_step<VS, MX>(r0, 0, MX ? h : 0, fa, fb);
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    const uint8_t* sbuf = lds + LDS_SCALES_AT + ((s >> 1) & 1) * SCALES;
    lds_read<VS, MX>(o, lds + cur * LDS_CODES, sbuf, cur, li, h, 1, r1);
    // NVFP4: k-steps 0..3 from r0, the last decoding k-step 4 from r1.
    // MXFP8: k-step 0 from r0, then k-step 1 decoding k-step 2 from r1;
    // every k-step of the stage uses scale byte 2 cur + h.
    if constexpr (MX) {
      kstep<VS, MX>(acc, fa, fb, r0, 1, 2 * cur + h);
      kstep<VS, MX>(acc, fa, fb, r1, 0, 2 * cur + h);
    } else {
      kstep<VS, MX>(acc, fa, fb, r0, 1, 0);
      kstep<VS, MX>(acc, fa, fb, r0, 2, 1);
      kstep<VS, MX>(acc, fa, fb, r0, 3, 1);
      kstep<VS, MX>(acc, fa, fb, r1, 0, 2);
    }
    // every read of stage s has been issued; once they land its code buffer
    // takes stage s + 2, and after an odd stage its scale pair buffer takes
    // the pair after next (stages s + 3, s + 4).  Stage s + 1 is in LDS once
    // only this iteration's DMAs can still be in flight.
    wait_lgkmcnt0();
    if (s + 2 < nst) {
      if (cur && s + 3 < nst) {
        lds_issue_scales<MX>(o, lbase + LDS_SCALES_AT + ((s >> 1) & 1) * SCALES, (uint32_t)(s + 3));
        lds_issue_codes<VS>(o, lbase + cur * LDS_CODES, (uint32_t)(s + 2));
        wait_vmcnt<NC + NS>();
      } else {
        lds_issue_codes<VS>(o, lbase + cur * LDS_CODES, (uint32_t)(s + 2));
        wait_vmcnt<NC>();
      }
    } else {
      wait_vmcnt<0>();
    }
    if (s + 1 < nst)
      lds_read<VS, MX>(o, lds + (cur ^ 1) * LDS_CODES,
                       lds + LDS_SCALES_AT + (((s + 1) >> 1) & 1) * SCALES, cur ^ 1, li, h, 0, r0);
    // the rest of the stage; the last k-step decodes k-step 0 of stage s + 1
    // (unused after the last stage)
    if constexpr (MX) {
      kstep<VS, MX>(acc, fa, fb, r1, 1, 2 * cur + h);
      kstep<VS, MX>(acc, fa, fb, r0, 0, 2 * (cur ^ 1) + h);
    } else {
      kstep<VS, MX>(acc, fa, fb, r1, 1, 2);
      kstep<VS, MX>(acc, fa, fb, r1, 2, 3);
      kstep<VS, MX>(acc, fa, fb, r1, 3, 3);
      kstep<VS, MX>(acc, fa, fb, r0, 0, 0);
    }
  }
  // per-row epilogue scales into the last 512 bytes of LDS (every read of
  // the K loop has landed: the final k-steps consumed them)
  float* s_rowscale = reinterpret_cast<float*>(lds + lds_wave<MX>() - 512);
  wait_lgkmcnt0();
  s_rowscale[lane] = rs0;
  s_rowscale[lane + 64] = rs1;
  __syncthreads();  // s_rowscale (written by this wave) is visible
  // Stores through a buffer resource over the tile's rows: the range check
  // drops rows past the tile's last and a huge offset drops columns past n,
  // so no store needs a branch.  Lane (li, h) holds, for slab i and
  // accumulator entry 4q + w, row 32i + 8q + 4h + w and column 32j + li; the
  // four rows' scales come in one 16-byte LDS read.
  if (p.n < ((int64_t)1 << 22)) {
    const uint32_t nb = (uint32_t)p.n * 4u;  // bytes per output row
    const __amdgpu_buffer_rsrc_t ry = out_rsrc(p.y + row_lo * p.n, (row_hi - row_lo) * p.n * 4);
    uint32_t vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      vb[j] = (n0 + 32 * j + li < p.n) ? (uint32_t)(4 * h) * nb + (uint32_t)(n0 + 32 * j + li) * 4u
                                        : 0x80000000u;
    f32x4 sc4[4][4];
#pragma unroll
    for (int i = 0; i < VS; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sc4[i][q] = *reinterpret_cast<const f32x4*>(s_rowscale + 32 * i + 8 * q + 4 * h);
    if constexpr (SW) {
      // SwiGLU epilogue: accumulator slabs 0-1 hold gate columns n0 + 32 j +
      // li, slabs 2-3 the up columns of the same H columns.  g and u are the
      // products the plain epilogue would store as Y; H[row, n0 + 32 j + li]
      // = swiglu(g, u) as bf16.  Rows past the tile fall outside the store
      // resource and columns past f get an out-of-range offset; each row's
      // largest |h| over the tile's columns (a 32-lane maximum over li) goes
      // to amax[row] by an atomic maximum of the bit pattern (order-free).
      const int64_t f = p.n / 2;
      const uint32_t hrow = (uint32_t)f * 2u;  // bytes per H row
      const __amdgpu_buffer_rsrc_t rh =
          out_rsrc(reinterpret_cast<float*>(p.h + row_lo * f), (row_hi - row_lo) * f * 2);
      uint32_t vh[2];
      bool cok[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        cok[j] = n0 + 32 * j + li < f;
        vh[j] = cok[j] ? (uint32_t)(4 * h) * hrow + (uint32_t)(n0 + 32 * j + li) * 2u : 0x80000000u;
      }
#pragma unroll
      for (int i = 0; i < VS; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float g = acc[i][j][4 * q + w] * sc4[i][q][w];
              const float u = acc[i][j + 2][4 * q + w] * sc4[i][q][w];
              const uint32_t b = swiglu_bf16(g, u);
              __builtin_amdgcn_raw_buffer_store_b16((unsigned short)b, rh,
                                                    vh[j] + (uint32_t)(32 * i + 8 * q + w) * hrow, 0, 2);
              m = max(m, cok[j] ? (b & 0x7FFFu) : 0u);
            }
            m = group_max_u32<32>(m);
            const int64_t row = row_lo + 32 * i + 8 * q + 4 * h + w;
            if (li == 0 && row < row_hi) atomicMax(reinterpret_cast<unsigned int*>(p.amax + row), m << 16);
          }
      return;
    }
    if ((p.n & 3) == 0) {
      // Through LDS, so every store writes 16 bytes and a store instruction
      // covers two whole 512-byte row segments: slab by slab, the scaled
      // values go to LDS rows of 544 bytes (the 32-byte pad puts the lane
      // halves' rows on disjoint banks), then lane L reads 16 bytes of row
      // 2t + L / 32 and stores them.  Four times fewer store instructions than
      // one value per lane, so the wave rarely stalls on its count of
      // outstanding memory operations.
      constexpr int RS = 544;
      float* t = reinterpret_cast<float*>(lds);
      const int rr = lane >> 5, cc = lane & 31;
      const int64_t col = n0 + 4 * cc;
      const uint32_t vc = col < p.n ? (uint32_t)col * 4u : 0x80000000u;
#pragma unroll
      for (int i = 0; i < VS; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t[((8 * q + 4 * h + w) * RS + (32 * j + li) * 4) / 4] = acc[i][j][4 * q + w] * sc4[i][q][w];
        wave_lds_sync();  // the slab's values are in LDS for every lane
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int r = 2 * u + rr;
          const f32x4 v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(t) + r * RS + cc * 16);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry,
                                                 vc + (uint32_t)(32 * i + r) * nb, 0, 2);
        }
        wave_lds_sync();  // the slab's reads are done before the next slab's writes
      }
      return;
    }
    if (row_hi - row_lo == 128 && n0 + 128 <= p.n) {
      // whole tile: the row offset is wave-uniform (scalar offset), the
      // column step an immediate
      const uint32_t vl = (uint32_t)(4 * h) * nb + (uint32_t)(n0 + li) * 4u;
#pragma unroll
      for (int i = 0; i < VS; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t ro = (uint32_t)(32 * i + 8 * q + w) * nb;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __builtin_bit_cast(uint32_t, acc[i][j][4 * q + w] * sc4[i][q][w]), ry, vl + 128 * j,
                  ro, 2);
          }
      return;
    }
#pragma unroll
    for (int i = 0; i < VS; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t ro = (uint32_t)(32 * i + 8 * q + w) * nb;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store_nt(ry, acc[i][j][4 * q + w] * sc4[i][q][w], vb[j] + ro);
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < VS; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lrow = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t row = row_lo + lrow;
      if (row >= row_hi) continue;
      const float sc = s_rowscale[lrow];
      float* yr = p.y + row * p.n;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + 32 * j + li;
        if (col < p.n) __builtin_nontemporal_store(acc[i][j][r] * sc, yr + col);
      }
    }
  }
}

// One 128 x 128 tile per one-wave block.  MX: operands are MXFP8 (E4M3
// codes, one byte per element; E8M0 scales per 32) and there is no outer
// scale (a_s, b_s unused).
template <bool MX, bool SW = false>
__device__ __forceinline__ void lds_tile(const GemmArgs& p, uint8_t* s_lds) {
  // SW: a tile is 64 columns of H, its B slabs the 64 gate rows (0-1) and
  // the 64 up rows (2-3) of those columns
  constexpr int BM = 128, BN = SW ? 64 : 128;
  static_assert(SCHED_LDS_WORDS * 4 <= LDS_CODES, "tile schedule must fit a code buffer");
  int32_t* s_prefix = reinterpret_cast<int32_t*>(s_lds + LDS_CODES);

  const int lane = threadIdx.x;
  const int h = lane >> 5, li = lane & 31;

  TileRange tr;
  if (!schedule_tile<BM, BN>(p.t, lane, s_prefix, tr)) return;  // block-uniform
  const int64_t row_lo = tr.row_lo, row_hi = tr.row_hi, n0 = tr.n0;
  const int g = tr.g;
  const int64_t rowb = MX ? p.k : p.k / 2, rows_s = MX ? p.k / 32 : p.k / 16;

  // Source A rows of the tile's 128 output rows: lane l looks up rows l and
  // 64 + l (two independent loads), every other lane's rows come by shuffle.
  const int32_t src0 = (int32_t)gathered_row(p.row_index, p.a_rows, row_lo + lane, row_hi);
  const int32_t src1 = (int32_t)gathered_row(p.row_index, p.a_rows, row_lo + 64 + lane, row_hi);
  auto src_of = [&](int half, int l) -> int64_t { return __shfl(half ? src1 : src0, l, 64); };

  LdsOperands o;
  o.aq = make_rsrc(p.a_q, p.a_rows * rowb);
  o.as = make_rsrc(p.a_sb, p.a_rows * rows_s);
  o.bq = make_rsrc(p.b_q + (int64_t)g * p.n * rowb, p.n * rowb);
  o.bs = make_rsrc(p.b_sb + (int64_t)g * p.n * rows_s, p.n * rows_s);
  o.avalid = o.bvalid = 0u;
  // DMA lanes: codes of row 16u + lane / 4 (chunk (lane & 3) ^ swz); scales
  // of row lane & 31 of slab 2q + lane / 32 (16 bytes: a stage pair).  Rows
  // that do not exist get an offset past the end of the operand, which the
  // buffer range check turns into no read.
  const uint32_t OOB = 0x80000000u;
  const int cr = lane >> 2, cc = lane & 3;
  // B row of row x of slab i, -1 past the weight (SW: gate rows n0 + 32 i + x
  // for slabs 0-1, up rows f + n0 + 32 (i - 2) + x for slabs 2-3)
  auto brow = [&](int i, int x) -> int64_t {
    if (SW) {
      const int64_t f = p.n / 2, c = n0 + 32 * (i & 1) + x;
      return c < f ? (i >= 2 ? f + c : c) : -1;
    }
    const int64_t c = n0 + 32 * i + x;
    return c < p.n ? c : -1;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int lr = 16 * u + cr;
      const uint32_t chunk = (uint32_t)((cc ^ lds_swz(lr)) * 16);
      const int64_t r = src_of(i >= 2, (32 * i + lr) & 63);
      o.aoff[i][u] = r >= 0 ? (uint32_t)(r * rowb) + chunk : OOB;
      const int64_t c = brow(i, lr);
      o.boff[i][u] = c >= 0 ? (uint32_t)(c * rowb) + chunk : OOB;
    }
    if (src_of(i >= 2, (32 * i + li) & 63) >= 0) o.avalid |= 1u << i;
    if (brow(i, li) >= 0) o.bvalid |= 1u << i;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t r = q ? src1 : src0;
    o.asoff[q] = r >= 0 ? (uint32_t)(r * rows_s) : OOB;
    const int64_t c = brow(2 * q + (lane >> 5), lane & 31);
    o.bsoff[q] = c >= 0 ? (uint32_t)(c * rows_s) : OOB;
  }
  // this lane's two epilogue row scales (rows lane and lane + 64), written to
  // LDS after the K loop
  // (MXFP8 rows without a source decode to exact zeros: their codes are masked)
  const float sbw = MX ? 1.0f : p.b_s[g];
  const float rs0 = MX ? 1.0f : (src0 >= 0 ? p.a_s[src0] : 0.0f) * sbw;
  const float rs1 = MX ? 1.0f : (src1 >= 0 ? p.a_s[src1] : 0.0f) * sbw;
  const int vslabs = (int)min((int64_t)4, (row_hi - row_lo + 31) / 32);
  switch (vslabs) {
    case 4: lds_body<4, MX, SW>(p, o, s_lds, h, li, lane, row_lo, row_hi, n0, rs0, rs1); break;
    case 3: lds_body<3, MX, SW>(p, o, s_lds, h, li, lane, row_lo, row_hi, n0, rs0, rs1); break;
    case 2: lds_body<2, MX, SW>(p, o, s_lds, h, li, lane, row_lo, row_hi, n0, rs0, rs1); break;
    default: lds_body<1, MX, SW>(p, o, s_lds, h, li, lane, row_lo, row_hi, n0, rs0, rs1); break;
  }
}

__global__ __launch_bounds__(64) void gemm_lds_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[lds_wave<false>()];
  lds_tile<false>(p, s_lds);
}

__global__ __launch_bounds__(64) void gemm_lds_swiglu_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[lds_wave<false>()];
  lds_tile<false, true>(p, s_lds);
}

__global__ __launch_bounds__(64) void mxfp8_gemm_lds_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[lds_wave<true>()];
  lds_tile<true>(p, s_lds);
}

// The MXFP8 GEMM on the one-wave LDS tile kernel when the shape allows it (k
// a multiple of 128: whole stage pairs; 16-byte aligned codes, 4-byte aligned
// scale rows; operands under 2 GiB); returns false otherwise.
bool launch_mxfp8_lds(const GemmArgs& a, bool grouped, hipStream_t stream) {
  GemmArgs p = a;
  const int64_t lim = (int64_t)1 << 31;
  if (p.k <= 0 || p.k % 128 != 0 || p.a_rows <= 0 || p.a_rows * p.k >= lim || p.n * p.k >= lim)
    return false;
  if (!nvfp4host::aligned(p.a_q, 16) || !nvfp4host::aligned(p.b_q, 16) ||
      !nvfp4host::aligned(p.a_sb, 4) || !nvfp4host::aligned(p.b_sb, 4))
    return false;
  const int64_t blocks = plan_tiles<128, 128>(p.t, p.n, grouped);
  hipLaunchKernelGGL(mxfp8_gemm_lds_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, p);
  return true;
}

template <int TM, int TN>
static void launch_gemm_rd(const GemmArgs& a, bool grouped, hipStream_t stream) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  GemmArgs p = a;
  const int64_t blocks = plan_tiles<BM, BN>(p.t, p.n, grouped, 4, p.row_index != nullptr);
  const bool fast = (p.k % BK) == 0 && nvfp4host::aligned(p.a_q, 16) &&
                    nvfp4host::aligned(p.b_q, 16) && nvfp4host::aligned(p.a_sb, 4) &&
                    nvfp4host::aligned(p.b_sb, 4);
  // the LDS path addresses operands with 32-bit buffer offsets
  const int64_t lim = (int64_t)1 << 31;
  const bool lds_ok = TM == 4 && TN == 4 && p.k % 256 == 0 && p.a_rows > 0 &&
                      p.a_rows * (p.k / 2) < lim && p.n * (p.k / 2) < lim;
  if (fast && lds_ok)
    hipLaunchKernelGGL(gemm_lds_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, p);
  else if (fast)
    hipLaunchKernelGGL((gemm_rd_kernel<TM, TN, true>), dim3((unsigned)blocks), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_rd_kernel<TM, TN, false>), dim3((unsigned)blocks), dim3(64), 0, stream, p);
}

// Y = 0 for k == 0 (no operand bytes to read).
__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ y, int64_t n_elems) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_elems; i += (int64_t)gridDim.x * 256)
    y[i] = 0.0f;
}

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
  if (m > ((int64_t)1 << 31) || n > ((int64_t)1 << 31) || k > ((int64_t)1 << 24) ||
      !nvfp4::tile_grid_ok(m, 0, n))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_sb, 16) || !aligned(b_sb, 16) ||
      !aligned(y, 16) || !aligned(a_s, 4) || !aligned(b_s, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.e4m3_codes(a_sb, m * (k / 16));
    chk.f32_finite(a_s, m);
    chk.e4m3_codes(b_sb, n * (k / 16));
    chk.f32_finite(b_s, 1);
    if ((st = chk.result())) return st;
  }
#endif
  hipStream_t str = (hipStream_t)stream;
  if (k == 0) {
    hipLaunchKernelGGL(nvfp4::zero_rows_kernel, dim3(1024), dim3(256), 0, str, y, m * n);
    return nvfp4host::launch_status();
  }
  nvfp4::GemmArgs p{};
  p.a_q = a_q; p.a_sb = a_sb; p.a_s = a_s; p.a_rows = m;
  p.row_index = nullptr; p.t.m_total = m; p.t.offsets = nullptr; p.t.groups = 1;
  p.b_q = b_q; p.b_sb = b_sb; p.b_s = b_s; p.n = n; p.k = k; p.y = y;
  if (!nvfp4::launch_gemm_skinny(p, false, str)) nvfp4::launch_gemm_rd<4, 4>(p, false, str);
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
      k > ((int64_t)1 << 24) || !nvfp4::tile_grid_ok(m_total, groups, n))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_sb, 16) || !aligned(b_sb, 16) ||
      !aligned(y, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(offsets, 4) ||
      !aligned(row_index, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.e4m3_codes(a_sb, a_rows * (k / 16));
    chk.f32_finite(a_s, a_rows);
    chk.e4m3_codes(b_sb, groups * n * (k / 16));
    chk.f32_finite(b_s, groups);
    chk.offsets(offsets, groups);
    if ((st = chk.result())) return st;
  }
#endif
  hipStream_t str = (hipStream_t)stream;
  nvfp4::GemmArgs p{};
  p.a_q = a_q; p.a_sb = a_sb; p.a_s = a_s; p.a_rows = a_rows;
  p.row_index = row_index; p.t.m_total = m_total; p.t.offsets = offsets; p.t.groups = (int)groups;
  p.b_q = b_q; p.b_sb = b_sb; p.b_s = b_s; p.n = n; p.k = k; p.y = y;
  // k == 0 needs no special case: the K loop is empty and the epilogue writes
  // zeros to exactly the rows the groups own
  if (!nvfp4::launch_gemm_skinny(p, true, str)) nvfp4::launch_gemm_rd<4, 4>(p, true, str);
  return nvfp4host::launch_status();
}

extern "C" int nvfp4_grouped_gemm_swiglu(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s,
                                         int64_t a_rows, const int32_t* row_index, int64_t m_total,
                                         const int32_t* offsets, int64_t groups, const uint8_t* b_q,
                                         const uint8_t* b_sb, const float* b_s, int64_t f, int64_t k,
                                         uint16_t* h, float* amax, void* stream) {
  if (groups < 1 || a_rows < 0 || m_total < 0 || f < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k == 0 || k % 256 != 0 || groups > nvfp4::MAX_GROUPS) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (m_total == 0 || f == 0) return NVFP4_SUCCESS;
  if (!offsets || !h || !amax || !b_s || !b_q || !b_sb) return NVFP4_ERROR_INVALID_VALUE;
  if (a_rows > 0 && (!a_q || !a_sb || !a_s)) return NVFP4_ERROR_INVALID_VALUE;
  if (!row_index && a_rows < m_total) return NVFP4_ERROR_INVALID_VALUE;
  const int64_t lim = (int64_t)1 << 31;
  if (m_total > lim || a_rows > lim || 2 * f >= ((int64_t)1 << 22) || k > ((int64_t)1 << 24) ||
      a_rows * (k / 2) >= lim || 2 * f * (k / 2) >= lim || !nvfp4::tile_grid_ok(m_total, groups, f))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_sb, 16) || !aligned(b_sb, 16) ||
      !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(offsets, 4) || !aligned(row_index, 4) ||
      !aligned(h, 2) || !aligned(amax, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.e4m3_codes(a_sb, a_rows * (k / 16));
    chk.f32_finite(a_s, a_rows);
    chk.e4m3_codes(b_sb, groups * 2 * f * (k / 16));
    chk.f32_finite(b_s, groups);
    chk.offsets(offsets, groups);
    if ((st = chk.result())) return st;
  }
#endif
  hipStream_t str = (hipStream_t)stream;
  // the row maxima are atomic maxima over the column tiles: start from zero
  // (a fill kernel, so the sequence can be captured in a graph)
  const int64_t zb = (m_total + 255) / 256;
  hipLaunchKernelGGL(nvfp4::zero_rows_kernel, dim3((unsigned)(zb < 1024 ? zb : 1024)), dim3(256), 0,
                     str, amax, m_total);
  nvfp4::GemmArgs p{};
  p.a_q = a_q; p.a_sb = a_sb; p.a_s = a_s; p.a_rows = a_rows;
  p.row_index = row_index; p.t.m_total = m_total; p.t.offsets = offsets; p.t.groups = (int)groups;
  p.b_q = b_q; p.b_sb = b_sb; p.b_s = b_s; p.n = 2 * f; p.k = k; p.y = nullptr;
  p.h = h; p.amax = amax;
  const int64_t blocks = nvfp4::plan_tiles<128, 64>(p.t, f, true);
  hipLaunchKernelGGL(nvfp4::gemm_lds_swiglu_kernel, dim3((unsigned)blocks), dim3(64), 0, str, p);
  return nvfp4host::launch_status();
}
