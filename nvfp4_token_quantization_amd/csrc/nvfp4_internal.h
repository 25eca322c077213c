// nvfp4_internal.h -- device helpers and host plumbing shared by the kernels
// of libnvfp4.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 hp16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// streaming 16-byte load (each input byte is read exactly once)
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// max of the 16 bf16 magnitudes held in two uint4 (as bf16 bit patterns)
__device__ __forceinline__ uint32_t block_amax_bits(const uint4& a, const uint4& b) {
  const uint32_t M = 0x7FFF7FFFu;
  u16x2 w[8];
  uint32_t t[8] = {a.x & M, a.y & M, a.z & M, a.w & M, b.x & M, b.y & M, b.z & M, b.w & M};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = __builtin_bit_cast(u16x2, t[i]);
  u16x2 m0 = __builtin_elementwise_max(__builtin_elementwise_max(w[0], w[1]),
                                       __builtin_elementwise_max(w[2], w[3]));
  u16x2 m1 = __builtin_elementwise_max(__builtin_elementwise_max(w[4], w[5]),
                                       __builtin_elementwise_max(w[6], w[7]));
  u16x2 m = __builtin_elementwise_max(m0, m1);
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// max of the 8 bf16 magnitudes held in one uint4 (as a bf16 bit pattern)
__device__ __forceinline__ uint32_t half_amax_bits(const uint4& a) {
  const uint32_t M = 0x7FFF7FFFu;
  const u16x2 m = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, a.x & M), __builtin_bit_cast(u16x2, a.y & M)),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, a.z & M), __builtin_bit_cast(u16x2, a.w & M)));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// ------------------------------------------------------------ E4M3 codec --
// RNE_SAT onto E4M3 (OCP FN, bias 7, max 448) for v >= 0 or +inf: returns
// the code and stores its exact value in `val`.  Values at or above 448 (and
// NaN) saturate; below 2^-6 the grid is the subnormal step 2^-9 and
// round-to-nearest-even on v * 2^9 is exact; otherwise the fp32 mantissa is
// rounded to 3 bits with ties to even (a carry moves into the exponent), and
// the rounded fp32 pattern is itself the value.  Branch-free: the candidates
// are formed and one selected.
__device__ __forceinline__ uint32_t e4m3_round(float v, float& val) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
  const float sub = __builtin_rintf(__builtin_fminf(v, 1.0f) * 512.0f);
  const bool is_sub = v < 0.015625f, sat = !(v < 448.0f);
  val = sat ? 448.0f : (is_sub ? sub * 0.001953125f : __uint_as_float(r));
  const uint32_t c = is_sub ? (uint32_t)sub : (r >> 20) - (120u << 3);
  return sat ? 0x7Eu : c;
}

__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  float val;
  return e4m3_round(v, val);
}

// Exact fp32 value of an E4M3 code 0..0x7E.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  float sub = (float)m * 0.001953125f;  // m * 2^-9
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e ? nrm : sub;
}

// Per-row (or per-group) scale terms: S = fl32(amax / 2688), t = fl32(6 S)
// and rt = fl32(1 / t), each correctly rounded.  `fast` says whether the
// quotients a_b / t of this row may be formed from rt (t well inside the
// normal range, so no intermediate below overflows or underflows).
struct RowScale {
  float S, t, rt;
  bool fast;
};

__device__ __forceinline__ RowScale row_scale(float amax) {
  RowScale r;
  r.S = amax / 2688.0f;
  r.t = 6.0f * r.S;
  r.fast = r.t >= 0x1p-100f && r.t <= 0x1p100f;
  r.rt = r.fast ? 1.0f / r.t : 0.0f;
  return r;
}

// Block scale code and reciprocal of d = S * s_b for one block whose largest
// magnitude has the bf16 bit pattern amax_bits:
//   code = RNE_SAT_E4M3(fl32(a_b / t)),  inv = fl32(1 / fl32(S * s_b)).
// Both fp32 results are the correctly rounded ones, formed with fma
// corrections instead of full divisions:
//  - quotient: q = fl32(a * rt), r = a - q t (exact in an fma), v = fl32(q +
//    r rt).  With rt the correctly rounded 1/t this is the correctly rounded
//    a / t for every bf16 significand of a and every fp32 significand of t
//    (an exhaustive check over all 2^30 pairs; exponents only scale the
//    values while nothing under- or overflows).  A subnormal a gives a
//    quotient far below 2^-10, where the code is 0 either way; a quotient
//    that overflows gives NaN or inf, which saturates like the exact one.
//  - reciprocal: y0 = v_rcp_f32(d) (within 1 ulp), e = 1 - d y0 (exact in an
//    fma), inv = fl32(y0 + e y0): correctly rounded for every fp32
//    significand and every y0 within 1 ulp of 1/d except the significand of
//    all ones (an exhaustive check), which takes the full division, as do
//    d outside [2^-125, 2^121) and d = 0 (inv = 0 there).
__device__ __forceinline__ void block_scale(uint32_t amax_bits, const RowScale& rs, uint32_t& code,
                                            float& inv) {
  const float ab = __uint_as_float(amax_bits << 16);
  float v;
  if (rs.fast) {
    const float q = ab * rs.rt;
    v = __builtin_fmaf(__builtin_fmaf(-q, rs.t, ab), rs.rt, q);
  } else {
    v = ab / rs.t;
  }
  float sbv;
  code = e4m3_round(v, sbv);
  if (rs.S == 0.0f) code = 0u;
  const float d = rs.S * sbv;  // S == 0 gives d == 0 whatever sbv is
  const uint32_t db = __float_as_uint(d);
  if (__builtin_expect(db - 0x01000000u < 0x7C000000u - 0x01000000u && (db & 0x7FFFFFu) != 0x7FFFFFu, 1)) {
    const float y0 = __builtin_amdgcn_rcpf(d);
    inv = __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
  } else {
    inv = (d != 0.0f) ? 1.0f / d : 0.0f;
  }
}

// ------------------------------------------------------------ E2M1 codec --
// Two fp32 values -> two E2M1 codes in byte `sel` of `old` (src0 in the low
// nibble).  gfx950's converter with scale 1.0 rounds to nearest even with
// ties to the even code, saturates to +-6 (also for +-inf) and copies the
// sign (including -0 and negative denormals); the exhaustive sweep test
// checks this against the oracle for every fp32 bit pattern.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_encode2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// ---------------------------------------------------- wave-level max (u32) --
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Max over aligned groups of L lanes (L = 16, 32 or 64) of a wave64; every
// lane of a group receives the group's max.  DPP quad permutes and row
// mirrors inside each 16-lane row, ds_swizzle (xor 16) across row pairs and
// readlane across the two halves of the wave.
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  v = max(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = max(v, dpp_mov<0x140>(v));  // row_mirror
  if (L >= 32) v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  if (L >= 64) {
    uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    v = max(a, b);
  }
  return v;
}

// Orders one wave's LDS accesses around an exchange of values between its
// lanes: every LDS write before the call is visible to every lane's LDS reads
// after it, and reads before the call complete before later writes.  (A
// wave's LDS operations already execute in order; this keeps the compiler
// from reordering them across the exchange.)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Raw buffer resource over `bytes` bytes of the output at p (stride 0;
// accesses whose offset is at or past `bytes` are dropped), built from
// wave-uniform (readfirstlane) values so accesses through it need no
// per-lane resource loop.  readfirstlane returns int: the halves are kept as
// uint32 so the low word is zero-extended, never sign-extended, into the
// 64-bit base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(float* p, int64_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int num = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, num,
                                           0x00020000);
}

}  // namespace nvfp4

// ------------------------------------------------------------- host side --
namespace nvfp4host {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Returns NVFP4_SUCCESS when the current device is gfx950 (cached per device).
int check_arch();

// Compute units of the current device (cached per device).
int num_cus();

// Rate of the device's constant wall clock (wall_clock64) in kHz (cached per
// device).
int64_t wall_clock_khz();

// Maps the last HIP launch error to a status.
int launch_status();

}  // namespace nvfp4host

#if NVFP4_CHECKED
// Device-side precondition checks of the checked build (checks.hip).  The
// constructor takes a library-wide lock and clears the violation flag on
// `stream`; each method launches one validation kernel there; result()
// waits for the stream and returns NVFP4_SUCCESS, NVFP4_ERROR_PRECONDITION
// or NVFP4_ERROR_LAUNCH, and releases the lock.  Null pointers and empty
// ranges check nothing.
namespace nvfp4check {

struct Checks {
  explicit Checks(hipStream_t s);
  ~Checks();
  void bf16_finite(const uint16_t* x, int64_t n);
  void f32_finite(const float* x, int64_t n, bool nonneg = false);
  void e4m3_codes(const uint8_t* c, int64_t n);  // no NaN code (0x7F, 0xFF)
  void e8m0_codes(const uint8_t* c, int64_t n);  // no NaN code (0xFF)
  void offsets(const int32_t* off, int64_t groups);  // off[0..groups] non-decreasing
  int result();

  hipStream_t stream;
  bool done = false;
};

}  // namespace nvfp4check
#endif
