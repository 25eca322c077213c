// gemm_common.h -- operands, exact FP4 x E4M3 -> fp16 decode and the
// kernel-selection hooks shared by the block-scaled GEMM kernels (gfx950).
#pragma once

#include "tile_sched.h"

namespace nvfp4 {

struct GemmArgs {
  const uint8_t* a_q;
  const uint8_t* a_sb;
  const float* a_s;
  int64_t a_rows;
  const int32_t* row_index;  // grouped only (nullable)
  const uint8_t* b_q;
  const uint8_t* b_sb;
  const float* b_s;
  int64_t n, k;
  float* y;
  TileGrid t;  // output rows / expert offsets and the launch plan
  // SwiGLU epilogue only (else null): bf16 H [m_total, n / 2] and its row
  // amax [m_total] (atomic maxima of the bit patterns; zeroed beforehand)
  uint16_t* h;
  float* amax;
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// E8M0 code -> the fp32 scale operand of the converter below (it uses only
// the exponent field: code e stands for 2^(e - 127), code 0 included)
__device__ __forceinline__ float e8m0_scale(uint32_t code) { return __uint_as_float(code << 23); }

// 8 MXFP8 elements (two dwords of E4M3 codes, byte order) times their block's
// power of two, as bf16: exact whenever the result is representable (an E4M3
// value has at most 4 significant bits and the scale only moves the exponent)
__device__ __forceinline__ bf16x8 mx_decode8(uint32_t w0, uint32_t w1, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return (bf16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int t) {
  return (t & 3) == 0 ? v.x : (t & 3) == 1 ? v.y : (t & 3) == 2 ? v.z : v.w;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));


// Raw buffer resource over `bytes` bytes at p (stride 0; loads whose VGPR
// offset is at or past `bytes` read nothing).
__device__ __forceinline__ i32x4 make_rsrc(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)p;
  return (i32x4){(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from rsrc[voff + soff] to LDS[lds + 16 * lane]
// (buffer_load ... lds: no VGPRs; rsrc, soff and lds must be wave-uniform,
// and the operand offsets 16-byte aligned).  Written as inline asm because
// the compiler's wait insertion cannot tell LDS buffers apart and would
// drain every DMA in flight before each ds_read; the asm clobbers memory
// and the callers wait explicitly (vmcnt before reading what a DMA wrote,
// lgkmcnt before a DMA overwrites what was read).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
// 4 bytes per lane from rsrc[voff + soff] to LDS[lds + 4 * lane] (as dma16)
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Rows few enough per expert (or per dense GEMM) that the weight stream, not
// the MFMAs, bounds the product: launches the split-K skinny kernel and
// returns true, or returns false when the shape is not one it takes (the
// caller then launches the tiled kernels).
bool launch_gemm_skinny(const GemmArgs& a, bool grouped, hipStream_t stream);

// The MXFP8 GEMM (a_q/b_q E4M3 codes, a_sb/b_sb E8M0 scales per 32, a_s and
// b_s unused) on the LDS tile kernel: returns false when the shape or the
// alignment is not one it takes.
bool launch_mxfp8_lds(const GemmArgs& a, bool grouped, hipStream_t stream);

}  // namespace nvfp4
