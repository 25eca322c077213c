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
  int slots;  // blocks that run at once on one XCD
};

// The block's output tile: rows [row_lo, row_hi) of expert g (0 when dense),
// columns from n0.
struct TileRange {
  int64_t row_lo, row_hi, n0;
  int g;
};

// Per-expert m-tile prefix of a contiguous per-expert layout, from the
// device offsets, by one wave of 64 lanes: s_prefix[g] = m-tiles of BM rows
// of the experts before g (s_prefix[G] = the total), and each expert's
// clamped row range [lo, hi) in the two arrays after the prefix (words
// MAX_GROUPS + 1 and 2 (MAX_GROUPS + 1) on; RANGES false: the prefix alone,
// MAX_GROUPS + 1 words).  Offsets are clamped to
// [0, m_total] and made non-decreasing, so bad metadata cannot address rows
// outside the output.  The caller synchronizes before reading s_prefix.
template <int BM, bool RANGES = true>
__device__ __forceinline__ void expert_tile_prefix(const int32_t* offsets, int G, int64_t m_total,
                                                   int lane, int32_t* s_prefix) {
  constexpr int GPT = MAX_GROUPS / 64;
  uint32_t* s_lo = reinterpret_cast<uint32_t*>(s_prefix + (MAX_GROUPS + 1));
  uint32_t* s_hi = reinterpret_cast<uint32_t*>(s_prefix + 2 * (MAX_GROUPS + 1));
  // every load first (indices clamped to the G + 1 entries), so they are in
  // flight together; a load under the per-entry condition below would wait
  // for each one in turn
  int32_t ov[GPT + 1];
#pragma unroll
  for (int i = 0; i <= GPT; ++i) ov[i] = offsets[min(lane * GPT + i, G)];
  int32_t local = 0;
  int32_t cnt[GPT];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int gg = lane * GPT + i;
    int32_t c = 0;
    if (gg < G) {
      int64_t lo = min(max((int64_t)ov[i], (int64_t)0), m_total);
      int64_t hi = min(max((int64_t)ov[i + 1], lo), m_total);
      c = (int32_t)((hi - lo + BM - 1) / BM);
      if (RANGES) {
        s_lo[gg] = (uint32_t)lo;  // m_total <= 2^31
        s_hi[gg] = (uint32_t)hi;
      }
    }
    cnt[i] = c;
    local += c;
  }
  int32_t incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  int32_t run = incl - local;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int gg = lane * GPT + i;
    if (gg <= G) s_prefix[gg] = run;
    run += cnt[i];
  }
  // the loop covers entries 0..MAX_GROUPS - 1; with G == MAX_GROUPS the
  // total (entry G) is the last lane's final running sum
  if (G == MAX_GROUPS && lane == 63) s_prefix[MAX_GROUPS] = run;
}

// The expert that owns global m-tile mt (mt < s_prefix[G]): the last g with
// s_prefix[g] <= mt, so experts without tiles are skipped.
__device__ __forceinline__ int find_expert(const int32_t* s_prefix, int G, int64_t mt) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_prefix[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// A readable int32 for the gathered-row load below when there is no index
// (its value is never used).
__device__ int32_t k_no_row_index[1] = {0};

// The A row that output row `out_row` of a tile with rows [.., row_hi)
// reads: row_index[out_row] (or out_row itself without an index), -1 when
// the output row is past the tile or the index falls outside [0, a_rows).
// The index load is unconditional and branch-free (clamped to the tile's
// last row, which exists; a dummy word without an index), so the loads of a
// lane's rows go out together instead of each waiting behind a branch.
__device__ __forceinline__ int64_t gathered_row(const int32_t* row_index, int64_t a_rows,
                                                int64_t out_row, int64_t row_hi) {
  const int64_t rr = min(out_row, row_hi - 1);
  const int32_t* src = row_index ? row_index + rr : k_no_row_index;
  const int32_t v = *src;
  const int64_t r = row_index ? (int64_t)v : rr;
  return (out_row < row_hi && r >= 0 && r < a_rows) ? r : -1;
}

// Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8);
// each XCD owns one region of an (8 / xcd_n) x xcd_n split of the tile grid
// so its L2 holds that region's A rows and B columns.  Inside a region, n runs
// fastest.  Grouped: every block derives the per-expert m-tile prefix from the
// device offsets (a wave scan into s_prefix) and binary-searches its expert.
// Returns false when the block has no tile (block-uniform).  Called by the
// whole block (one wave of 64 lanes).
template <int BM, int BN>
__device__ __forceinline__ bool schedule_tile(const TileGrid& t, int lane,
                                              int32_t* s_prefix /* SCHED_LDS_WORDS */,
                                              TileRange& out) {
  const int xcd = blockIdx.x % 8;
  const int64_t jloc = blockIdx.x / 8;
  const int xn = xcd % t.xcd_n, xm = xcd / t.xcd_n, XM = 8 / t.xcd_n;
  const int64_t npx = (t.tiles_n + t.xcd_n - 1) / t.xcd_n;
  const int64_t nlo = xn * npx, nhi = min((int64_t)t.tiles_n, nlo + npx);
  if (nlo >= nhi) return false;  // block-uniform
  const int64_t width = nhi - nlo;
  // Region tiles are issued in order; when the last round of a region would
  // leave more than half of the XCD's slots idle, its tiles are issued as
  // two halves of BM / 2 rows so that round takes about half as long.
  auto place = [&](int64_t mcount, int64_t& jf, int& hf) -> bool {
    const int64_t T = mcount * width;
    const int64_t tail = T % t.slots;
    const int64_t split = (tail != 0 && 2 * tail <= t.slots) ? tail : 0;
    const int64_t F = T - split;
    if (jloc < F) {
      jf = jloc;
      hf = -1;
      return true;
    }
    const int64_t hidx = jloc - F;
    if (hidx >= 2 * split) return false;
    jf = F + hidx / 2;
    hf = (int)(hidx & 1);
    return true;
  };
  int64_t jf = 0, mt, nt;
  int hf = -1;
  int64_t row_lo, row_hi;
  int g = 0;
  if (t.offsets) {
    const int G = t.groups;
    const uint32_t* s_lo = reinterpret_cast<const uint32_t*>(s_prefix + (MAX_GROUPS + 1));
    const uint32_t* s_hi = reinterpret_cast<const uint32_t*>(s_prefix + 2 * (MAX_GROUPS + 1));
    expert_tile_prefix<BM>(t.offsets, G, t.m_total, lane, s_prefix);
    __syncthreads();
    const int64_t total_mt = s_prefix[G];
    const int64_t mpx = (total_mt + XM - 1) / XM;
    const int64_t mcount = min(mpx, max(total_mt - xm * mpx, (int64_t)0));
    if (!place(mcount, jf, hf)) return false;  // block-uniform
    mt = xm * mpx + jf / width;
    nt = nlo + jf % width;
    g = find_expert(s_prefix, G, mt);
    const int64_t glo = (int64_t)s_lo[g];
    const int64_t ghi = (int64_t)s_hi[g];
    row_lo = glo + (mt - s_prefix[g]) * BM;
    row_hi = min(ghi, row_lo + BM);
  } else {
    const int64_t tiles_m = (t.m_total + BM - 1) / BM;
    const int64_t mpx = (tiles_m + XM - 1) / XM;
    const int64_t mcount = min(mpx, max(tiles_m - xm * mpx, (int64_t)0));
    if (!place(mcount, jf, hf)) return false;  // block-uniform
    mt = xm * mpx + jf / width;
    nt = nlo + jf % width;
    row_lo = mt * BM;
    row_hi = min(t.m_total, row_lo + BM);
  }
  if (hf >= 0) {  // half tile: rows [row_lo + (BM/2) hf, row_lo + (BM/2)(hf + 1))
    row_lo += (BM / 2) * hf;
    row_hi = min(row_hi, row_lo + BM / 2);
  }
  if (row_lo >= row_hi) return false;  // block-uniform (never for a consistent prefix)
  out.row_lo = row_lo;
  out.row_hi = row_hi;
  out.n0 = nt * BN;
  out.g = g;
  return true;
}

// Fill of an even split of `tiles` into `parts` ranges (1.0 = balanced).
static inline double split_fill(int64_t tiles, int parts) {
  const int64_t per = (tiles + parts - 1) / parts;
  return per > 0 ? (double)tiles / (double)(per * parts) : 1.0;
}

// Host launch plan for BM x BN tiles, `per_cu` blocks resident per CU (4
// one-wave blocks, or 1 four-wave block): fills tiles_n, xcd_n and slots and
// returns the number of blocks to launch.
template <int BM, int BN>
static int64_t plan_tiles(TileGrid& t, int64_t n, bool grouped, int per_cu = 4) {
  t.tiles_n = (int)((n + BN - 1) / BN);
  // upper bound on m-tiles (grouped: each group adds at most a partial tile;
  // the exact count is derived on the device from the offsets)
  const int64_t tiles_m = (t.m_total + BM - 1) / BM + (grouped ? t.groups : 0);
  // XCD split: grouped GEMMs split along M (B changes along M); dense GEMMs
  // take the split with the best balance, preferring more N regions.
  t.xcd_n = 1;
  if (!grouped) {
    double best = -1.0;
    for (int xn = 1; xn <= 8; xn *= 2) {
      const double f = split_fill(tiles_m, 8 / xn) * split_fill(t.tiles_n, xn);
      if (f >= best) { best = f; t.xcd_n = xn; }
    }
  }
  t.slots = (nvfp4host::num_cus() / 8) * per_cu;
  if (t.slots < 2) t.slots = 2;
  const int64_t per_xcd = ((tiles_m + (8 / t.xcd_n) - 1) / (8 / t.xcd_n)) *
                              ((t.tiles_n + t.xcd_n - 1) / t.xcd_n) +
                          t.slots / 2;  // room for the split tail
  return 8 * per_xcd;
}

}  // namespace nvfp4
