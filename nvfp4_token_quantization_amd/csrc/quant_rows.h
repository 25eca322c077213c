// quant_rows.h -- the per-row encode of the NVFP4 quantizers (gfx950): a
// row group held in registers by L lanes per row, its block and row amax,
// and the encode and stores of one row group.  Shared by the row kernels and
// the one-pass weight kernel (quantize.hip, weight_onepass.h).
//
// Method: the Miles page ("Towards Blackwell-Native 8-bit and 4-bit RL"),
// section 速读 (16 E2M1 values per E4M3 block scale under an FP32 outer
// scale) and section 单Token缩放的在线计算实现; the TRIAGE page, section
// 前置知识, for x_hat = S * s_b * Q_E2M1(x / (S * s_b)).
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

enum QuantMode { MODE_ROW = 0, MODE_AMAX_IN = 1, MODE_GROUP = 2 };

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Encode one half-block of 8 elements (a uint4 of bf16) with reciprocal
// `inv` into a dword of E2M1 codes.  When inv is +inf (d is a tiny denormal)
// x * inv would be NaN for x = +-0, so zeros are passed through unchanged.
__device__ __forceinline__ uint32_t encode_half(const uint4& a, float inv) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  float r[8];
  if (__builtin_expect(__builtin_isinf(inv), 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo = bf16lo(w[i]), hi = bf16hi(w[i]);
      r[2 * i] = (lo == 0.0f) ? lo : lo * inv;
      r[2 * i + 1] = (hi == 0.0f) ? hi : hi * inv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = bf16lo(w[i]) * inv;
      r[2 * i + 1] = bf16hi(w[i]) * inv;
    }
  }
  uint32_t q = 0;
  q = e2m1_encode2<0>(q, r[0], r[1]);
  q = e2m1_encode2<1>(q, r[2], r[3]);
  q = e2m1_encode2<2>(q, r[4], r[5]);
  q = e2m1_encode2<3>(q, r[6], r[7]);
  return q;
}

// The U half-blocks of one row group held by a lane, and the row's supplied
// amax (row or group) when there is one.  The amax load is issued before the
// row's data loads: vector memory counters retire in order, so waiting for
// the data then also covers the amax, and nothing forces a wait on a load
// issued later (the next group's prefetch).
template <int U>
struct RowData {
  uint4 d[U];
  float amax;
  int64_t gi;  // group of the row (MODE_GROUP)
};

template <int L, int U, int MODE>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t k,
                                          int nh, int64_t row, int j,
                                          const float* __restrict__ amax_src,
                                          int64_t rows_per_group, RowData<U>& r) {
  const bool row_ok = row < rows;
  if (MODE == MODE_AMAX_IN) {
    r.amax = row_ok ? amax_src[row] : 0.0f;
  } else if (MODE == MODE_GROUP) {
    r.gi = row_ok ? row / rows_per_group : 0;
    r.amax = row_ok ? amax_src[r.gi] : 0.0f;
  }
  const uint4* xr = reinterpret_cast<const uint4*>(x + (row_ok ? row : 0) * k);
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int h = j + L * i;
    r.d[i] = (row_ok && h < nh) ? ld_stream(xr + h) : make_uint4(0, 0, 0, 0);
  }
}

// Block amax of the half-block held by this lane and its partner (lane ^ 1).
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
  return max(v, dpp_mov<0xB1>(v));  // quad_perm [1,0,3,2]
}

// Encode and store one row group.  Must be called by all 64 lanes of the
// wave (block and row amax are cross-lane reductions).  The first `qskip`
// code dwords of the row are left unwritten (a caller writes them later).
template <int L, int U, int MODE>
__device__ __forceinline__ void encode_rows(const RowData<U>& r, int64_t rows, int64_t k, int nh,
                                            int64_t row, int j,
                                            const float* __restrict__ amax_src,
                                            int64_t rows_per_group, uint8_t* __restrict__ q,
                                            uint8_t* __restrict__ sb, float* __restrict__ s,
                                            int qskip = 0) {
  const bool row_ok = row < rows;
  uint32_t bmax[U];
  uint32_t rmax = 0;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    bmax[i] = pair_max(half_amax_bits(r.d[i]));
    rmax = max(rmax, bmax[i]);
  }
  const float amax = (MODE == MODE_ROW) ? __uint_as_float(group_max_u32<L>(rmax) << 16) : r.amax;
  const RowScale rs = row_scale(amax);
  if (MODE != MODE_GROUP && row_ok && j == 0) s[row] = rs.S;
  // the group's first row also stores its outer scale (when asked to)
  if (MODE == MODE_GROUP && s && row_ok && j == 0 && row == r.gi * rows_per_group) s[r.gi] = rs.S;
  // Both lanes of a pair hold the same blocks; for slots (i, i + 1) the even
  // lane derives block i's scale and the odd lane block i + 1's, and a DPP
  // swap hands each lane the other result (an odd last slot is derived by
  // both).  Every lane runs this part, so the swaps see their partners.
  uint32_t code[U];
  float inv[U];
  const bool odd = (j & 1) != 0;
#pragma unroll
  for (int i = 0; i + 1 < U; i += 2) {
    uint32_t c;
    float v;
    block_scale(odd ? bmax[i + 1] : bmax[i], rs, c, v);
    const uint32_t c_p = dpp_mov<0xB1>(c);
    const float v_p = __uint_as_float(dpp_mov<0xB1>(__float_as_uint(v)));
    code[i] = odd ? c_p : c;
    inv[i] = odd ? v_p : v;
    code[i + 1] = odd ? c : c_p;
    inv[i + 1] = odd ? v : v_p;
  }
  if (U & 1) block_scale(bmax[U - 1], rs, code[U - 1], inv[U - 1]);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + (row_ok ? row : 0) * (k / 2));
  uint8_t* sr = sb + (row_ok ? row : 0) * (k / 16);
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int h = j + L * i;
    if (row_ok && h < nh) {
      if (h >= qskip) qr[h] = encode_half(r.d[i], inv[i]);
      if (!odd) sr[h >> 1] = (uint8_t)code[i];
    }
  }
}

}  // namespace nvfp4
