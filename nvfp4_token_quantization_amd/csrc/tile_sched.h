// tile_sched.h -- block -> output-tile mapping shared by the GEMM kernels
// (dense and grouped, gfx950): XCD-aware regions, device-side expert tile
// prefix from the offsets, and the split of a region's last partial round.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

constexpr int MAX_GROUPS = 1024;
// int32 words of LDS schedule_tile needs: the expert m-tile prefix, then each
// expert's clamped row range [lo, hi) (so the block's expert bounds come from
// LDS, not from a second dependent read of the offsets in memory)
constexpr int SCHED_LDS_WORDS = 3 * (MAX_GROUPS + 1);

// What the mapping needs: the output rows (dense) or the device offsets of a
// contiguous per-expert layout (grouped), and the host's launch plan.
struct TileGrid {
  int64_t m_total;          // grouped: output rows; dense: m
  const int32_t* offsets;   // grouped only (nullptr: dense)
  int groups;               // grouped only
  int tiles_n;
  int xcd_n;  // XCD regions along N (8 / xcd_n along M)
  int cost_split;  // grouped, up to 256 experts: M regions bounded by estimated tile cost
  int slots;  // blocks that run at once on one XCD
};

// The block's output tile: rows [row_lo, row_hi) of expert g (0 when dense),
// columns from n0.
struct TileRange {
  int64_t row_lo, row_hi, n0;
  int g;
};

// Per-expert m-tile prefix of a contiguous per-expert layout, from the
// device offsets, by one wave of 64 lanes: s_prefix[e] = m-tiles of BM rows
// of the experts before e (s_prefix[G] = the total), and each expert's
// clamped row range [s_lo[e], s_hi[e]).  Offsets are clamped to [0, m_total]
// and made non-decreasing, so bad metadata cannot address rows outside the
// output.  Four 64-expert segments per round of coalesced loads (lane l reads
// offsets e and e + 1 of expert e = 64 i + l), a wave scan per segment
// (segments past G are skipped); all arithmetic in 32 bits (offsets are
// int32).  The caller synchronizes before reading the arrays.
// Inclusive prefix sum over the 64 lanes of a wave in DPP moves (no LDS
// permutes): shifts right by 1, 2, 4 and 8 lanes inside each 16-lane row
// (lanes shifted in from outside the row read 0), then lane 15's sum added to
// rows 1 and 3 (row_bcast:15, row mask 0b1010) and lane 31's to rows 2 and 3
// (row_bcast:31, row mask 0b1100); rows outside a mask add 0.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
  v = wave_incl_scan(v);
  return __builtin_amdgcn_readlane(v, 63);
}

template <int BM>
__device__ __forceinline__ void expert_tile_prefix(const int32_t* offsets, int G, int64_t m_total,
                                                   int lane, int32_t* s_prefix, int32_t* s_lo,
                                                   int32_t* s_hi) {
  const int32_t mt = (int32_t)min(m_total, (int64_t)0x7FFFFFFF);
  int32_t carry = 0;
  for (int e0 = 0; e0 < G; e0 += 256) {
    int32_t o0[4], o1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // every load first, so they are in flight together
      const int e = e0 + 64 * i + lane;
      if (e0 + 64 * i < G) {
        o0[i] = offsets[min(e, G)];
        o1[i] = offsets[min(e + 1, G)];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (e0 + 64 * i >= G) break;
      const int e = e0 + 64 * i + lane;
      const int32_t lo = min(max(o0[i], 0), mt);
      const int32_t hi = min(max(o1[i], lo), mt);
      const int32_t c = e < G ? (int32_t)(((uint32_t)(hi - lo) + (BM - 1)) / BM) : 0;
      const int32_t incl = wave_incl_scan(c);
      if (e < G) {
        s_prefix[e] = carry + incl - c;
        s_lo[e] = lo;
        s_hi[e] = hi;
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (lane == 0) s_prefix[G] = carry;
}

// The expert that owns m-tile mt < s_prefix[G]: the number of experts whose
// first m-tile is at or before mt, less one (experts without m-tiles share
// their first m-tile with the next expert that has one, so they are passed
// over).  Called by all 64 lanes of a wave.
__device__ __forceinline__ int find_expert(const int32_t* s_prefix, int G, int mt, int lane) {
  int count = 0;
  for (int e0 = 0; e0 < G; e0 += 256) {
    int32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + 64 * i < G) v[i] = s_prefix[min(e0 + 64 * i + lane, G)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + 64 * i < G) count += __popcll(__ballot(e0 + 64 * i + lane < G && v[i] <= mt));
  }
  return count - 1;
}

// The A row that output row `out_row` of a tile with rows [.., row_hi)
// reads: row_index[out_row] (or out_row itself without an index), -1 when
// the output row is past the tile or the index falls outside [0, a_rows).
// With an index the load is unconditional (clamped to the tile's last row,
// which exists), so the loads of a lane's rows go out together instead of
// each waiting behind a per-lane branch.
__device__ __forceinline__ int64_t gathered_row(const int32_t* row_index, int64_t a_rows,
                                                int64_t out_row, int64_t row_hi) {
  // without an index (a kernel argument, so the branch is uniform) there is
  // nothing to load: the A row is the output row
  if (!row_index) return (out_row < row_hi && out_row < a_rows) ? out_row : -1;
  const int64_t rr = min(out_row, row_hi - 1);
  const int64_t r = (int64_t)row_index[rr];
  return (out_row < row_hi && r >= 0 && r < a_rows) ? r : -1;
}

// Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8);
// each XCD owns one region of an (8 / xcd_n) x xcd_n split of the tile grid
// so its L2 holds that region's A rows and B columns.  Inside a region,
// grouped GEMMs run n fastest (an expert's m-tiles share its B panels);
// dense GEMMs run bands of 8 m-tiles, m fastest within a band.  Grouped:
// every block derives the per-expert m-tile prefix from the device offsets
// (a wave scan, in registers for up to 256 experts, else into s_prefix) and
// finds its expert by a ballot count.
// Returns false when the block has no tile (block-uniform).  Called by the
// whole block (one wave of 64 lanes).
template <int BM, int BN>
__device__ __forceinline__ bool schedule_tile(const TileGrid& t, int lane,
                                              int32_t* s_prefix /* SCHED_LDS_WORDS */,
                                              TileRange& out) {
  // tile counts and indices fit in 32 bits; 64-bit divisions by run-time
  // values are long software sequences here
  const int xcd = (int)(blockIdx.x % 8);
  const int jloc = (int)(blockIdx.x / 8);
  const int xn = xcd % t.xcd_n, xm = xcd / t.xcd_n, XM = 8 / t.xcd_n;
  const int npx = (t.tiles_n + t.xcd_n - 1) / t.xcd_n;
  const int nlo = xn * npx, nhi = min(t.tiles_n, nlo + npx);
  if (nlo >= nhi) return false;  // block-uniform
  const int width = nhi - nlo;
  // Region tiles are issued in order; when the last round of a region would
  // leave more than half of the XCD's slots idle, its tiles are issued as
  // two halves of BM / 2 rows so that round takes about half as long.
  auto place = [&](int mcount, int& jf, int& hf) -> bool {
    const int T = mcount * width;
    const int tail = T % t.slots;
    const int split = (tail != 0 && 2 * tail <= t.slots) ? tail : 0;
    const int F = T - split;
    if (jloc < F) {
      jf = jloc;
      hf = -1;
      return true;
    }
    const int hidx = jloc - F;
    if (hidx >= 2 * split) return false;
    jf = F + hidx / 2;
    hf = hidx & 1;
    return true;
  };
  int jf = 0, hf = -1, mt, nt;
  int64_t row_lo, row_hi;
  int g = 0;
  if (t.offsets && t.groups <= 256) {
    // Up to 256 experts: one round of offset loads, and the m-tile prefix,
    // the expert lookup and its row range stay in registers (no LDS round
    // trip, no barrier).  Same arithmetic as expert_tile_prefix and
    // find_expert: lo / hi the clamped row range of expert 64 i + lane, ex
    // the m-tiles of the experts before it; the expert's values come from its
    // lane by readlane.
    const int G = t.groups;
    const int32_t mtot = (int32_t)min(t.m_total, (int64_t)0x7FFFFFFF);
    int32_t o0[4], o1[4], lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0}, ex[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 64 * i + lane;
      if (64 * i < G) {
        o0[i] = t.offsets[min(e, G)];
        o1[i] = t.offsets[min(e + 1, G)];
      }
    }
    int32_t carry = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (64 * i >= G) break;
      const int e = 64 * i + lane;
      lo[i] = min(max(o0[i], 0), mtot);
      hi[i] = min(max(o1[i], lo[i]), mtot);
      const int32_t c = e < G ? (int32_t)(((uint32_t)(hi[i] - lo[i]) + (BM - 1)) / BM) : 0;
      const int32_t incl = wave_incl_scan(c);
      ex[i] = carry + incl - c;
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    const int total_mt = carry;
    int m0, mcount;
    if (t.cost_split) {
      // Regions of equal estimated cost rather than equal m-tile counts: a
      // partial expert tile runs fewer 32-row slabs but streams and decodes
      // the same B panel.  Costs in 1/20 of a full tile, from per-block
      // timing stamps (4 valid slabs, full or not, 20; 1, 2, 3 slabs 10, 13,
      // 17).  A region holds the m-tiles whose starting cost falls in its
      // 1/XM of the total, in expert order.
      int32_t cx[4] = {0, 0, 0, 0}, cn[4] = {0, 0, 0, 0};
      int64_t ccarry = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (64 * i >= G) break;
        const int e = 64 * i + lane;
        const int32_t rows = hi[i] - lo[i];
        const int32_t full = rows / BM, rem = rows - full * BM;
        const int32_t v = (rem + 31) / 32;
        const int32_t w = v == 0 ? 0 : (v == 1 ? 10 : (v == 2 ? 13 : (v == 3 ? 17 : 20)));
        const int32_t ce = e < G ? 20 * full + w : 0;
        const int32_t incl = wave_incl_scan(ce);
        cx[i] = (int32_t)ccarry + incl - ce;
        cn[i] = e < G ? full + (v > 0 ? 1 : 0) : 0;
        ccarry += __builtin_amdgcn_readlane(incl, 63);
      }
      auto tiles_before = [&](int64_t bound) -> int {
        int32_t s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (64 * i >= G) break;
          const int64_t d = bound - cx[i];
          const int32_t tb = d <= 0 ? 0 : (int32_t)min((d + 19) / 20, (int64_t)cn[i]);
          s += tb;
        }
        return wave_sum_i32(s);
      };
      m0 = tiles_before(ccarry * xm / XM);
      mcount = tiles_before(ccarry * (xm + 1) / XM) - m0;
    } else {
      const int mpx = (total_mt + XM - 1) / XM;
      m0 = xm * mpx;
      mcount = min(mpx, max(total_mt - xm * mpx, 0));
    }
    if (!place(mcount, jf, hf)) return false;  // block-uniform
    mt = m0 + jf / width;
    nt = nlo + jf % width;
    int count = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (64 * i < G) count += __popcll(__ballot(64 * i + lane < G && ex[i] <= mt));
    g = max(count - 1, 0);
    const int seg = g >> 6, ln = g & 63;
    int32_t lo_s = lo[0], hi_s = hi[0], ex_s = ex[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (seg == i) { lo_s = lo[i]; hi_s = hi[i]; ex_s = ex[i]; }
    row_lo = (int64_t)__builtin_amdgcn_readlane(lo_s, ln) +
             (int64_t)(mt - __builtin_amdgcn_readlane(ex_s, ln)) * BM;
    row_hi = min((int64_t)__builtin_amdgcn_readlane(hi_s, ln), row_lo + BM);
  } else if (t.offsets) {
    const int G = t.groups;
    int32_t* s_lo = s_prefix + (MAX_GROUPS + 1);
    int32_t* s_hi = s_prefix + 2 * (MAX_GROUPS + 1);
    expert_tile_prefix<BM>(t.offsets, G, t.m_total, lane, s_prefix, s_lo, s_hi);
    __syncthreads();
    const int total_mt = s_prefix[G];
    const int mpx = (total_mt + XM - 1) / XM;
    const int mcount = min(mpx, max(total_mt - xm * mpx, 0));
    if (!place(mcount, jf, hf)) return false;  // block-uniform
    mt = xm * mpx + jf / width;
    nt = nlo + jf % width;
    g = find_expert(s_prefix, G, mt, lane);
    row_lo = (int64_t)s_lo[g] + (int64_t)(mt - s_prefix[g]) * BM;
    row_hi = min((int64_t)s_hi[g], row_lo + BM);
  } else {
    const int tiles_m = (int)((t.m_total + BM - 1) / BM);
    const int mpx = (tiles_m + XM - 1) / XM;
    const int mcount = min(mpx, max(tiles_m - xm * mpx, 0));
    if (!place(mcount, jf, hf)) return false;  // block-uniform
    // bands of 8 m-tiles, every n-tile of the region per band, the band's
    // m-tiles fastest: an XCD's concurrent tiles then share fewer A rows and
    // B columns between them (4096 x 9728 x 2560: about 1% faster than n
    // fastest over the whole region)
    constexpr int GM = 8;
    const int band = jf / (GM * width), within = jf % (GM * width);
    const int bh = min(GM, mcount - band * GM);
    mt = xm * mpx + band * GM + within % bh;
    nt = nlo + within / bh;
    row_lo = (int64_t)mt * BM;
    row_hi = min(t.m_total, row_lo + BM);
  }
  if (hf >= 0) {  // half tile: rows [row_lo + (BM/2) hf, row_lo + (BM/2)(hf + 1))
    row_lo += (BM / 2) * hf;
    row_hi = min(row_hi, row_lo + BM / 2);
  }
  if (row_lo >= row_hi) return false;  // block-uniform (never for a consistent prefix)
  out.row_lo = row_lo;
  out.row_hi = row_hi;
  out.n0 = (int64_t)nt * BN;
  out.g = g;
  return true;
}

// Host check that a tiled launch's grid stays far below 2^31 blocks (tile
// indices are 32-bit, and a cost-bounded grouped plan launches up to twice
// the tiles): at most 2^28 tiles of 128 x 64 over the output rows plus one
// partial tile per group.  Only outputs far beyond device memory fail it.
static inline bool tile_grid_ok(int64_t m_total, int64_t groups, int64_t n) {
  return ((m_total + 127) / 128 + groups + 1) * ((n + 63) / 64 + 1) <= ((int64_t)1 << 28);
}

// Fill of an even split of `tiles` into `parts` ranges (1.0 = balanced).
static inline double split_fill(int64_t tiles, int parts) {
  const int64_t per = (tiles + parts - 1) / parts;
  return per > 0 ? (double)tiles / (double)(per * parts) : 1.0;
}

// Host launch plan for BM x BN tiles, `per_cu` blocks resident per CU (4
// one-wave blocks, or 1 four-wave block): fills tiles_n, xcd_n and slots and
// returns the number of blocks to launch.  `gathered`: a grouped GEMM reads
// its A rows through row_index.
template <int BM, int BN>
static int64_t plan_tiles(TileGrid& t, int64_t n, bool grouped, int per_cu = 4, bool gathered = true) {
  t.tiles_n = (int)((n + BN - 1) / BN);
  // upper bound on m-tiles (grouped: each group adds at most a partial tile;
  // the exact count is derived on the device from the offsets)
  const int64_t tiles_m = (t.m_total + BM - 1) / BM + (grouped ? t.groups : 0);
  // XCD split: grouped GEMMs split along M (B changes along M; an expert's
  // m-tiles share its B panels in one L2); dense GEMMs take the split with
  // the best balance, preferring more N regions.  A grouped GEMM that reads
  // A in place (no row_index) splits into 2 M halves x 4 N slices when N
  // divides evenly: an M range of partial and full expert tiles costs
  // unevenly (measured on the Zipf-routed down projection: the costliest of
  // 8 M regions holds 12% more work than the mean, 2.5% with 4 N slices), and
  // re-reading contiguous A rows once per N slice is cheap.  Gathered A rows
  // are scattered, and re-reading them cost more than the balance gained
  // (up projection +3%, down projection -3%).
  t.xcd_n = 1;
  t.cost_split = 0;
  if (grouped && !gathered && split_fill(t.tiles_n, 4) >= 0.9) t.xcd_n = 4;
  // Gathered grouped GEMMs (the up projection) keep whole M regions and
  // bound them by estimated cost instead (the schedule's register path, up
  // to 256 experts; the 128-row tile kernels, which run only a partial
  // tile's valid slabs): up projection 3.5% faster in same-box pairs.
  if (grouped && gathered && t.groups <= 256 && BM == 128) t.cost_split = 1;
  if (!grouped) {
    double best = -1.0;
    for (int xn = 1; xn <= 8; xn *= 2) {
      const double f = split_fill(tiles_m, 8 / xn) * split_fill(t.tiles_n, xn);
      if (f >= best) { best = f; t.xcd_n = xn; }
    }
  }
  t.slots = (nvfp4host::num_cus() / 8) * per_cu;
  if (t.slots < 2) t.slots = 2;
  // a cost-bounded region holds at most twice the mean m-tile count (no
  // tile costs less than half a full one), plus one
  const int64_t mreg = t.cost_split ? 2 * ((tiles_m + (8 / t.xcd_n) - 1) / (8 / t.xcd_n)) + 1
                                    : (tiles_m + (8 / t.xcd_n) - 1) / (8 / t.xcd_n);
  const int64_t per_xcd = mreg * ((t.tiles_n + t.xcd_n - 1) / t.xcd_n) + t.slots / 2;  // room for the split tail
  return 8 * per_xcd;
}

}  // namespace nvfp4
