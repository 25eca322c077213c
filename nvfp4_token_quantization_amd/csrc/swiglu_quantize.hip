// swiglu_quantize.hip -- SwiGLU over a fused gate|up projection followed by
// per-token NVFP4 quantization of its bf16 output, in one pass (gfx950).
//
// The pages' MoE layers fuse gate and up into one GEMM under one FP32 weight
// scale (Miles page, section 并行度与张量转换的一致性契约); the miniTE page
// (section Transformer Engine路径优化) names amax reuse and fusion as the way
// to cut the data preparation around the low-precision GEMMs.  Here the row
// amax of H = silu(gate) * up never leaves registers: the kernel that produces
// H also encodes it, so H is neither written nor read back unless the caller
// asks for the bf16 copy (for a backward pass).
//
// Per element: h = bf16(fl32(g * u / (1 + exp(-g)))) with the quotient formed
// in fp64 (g * u is exact there), so the fp32 value is the correctly rounded
// one except when the true value lies within ~1e-16 relative of an fp32
// rounding boundary.  An fp32 evaluation with a rounding test returns the
// same bf16 for all but about 1 element in 2000, which take the fp64 path.  The bf16 codes then follow exactly the per-token
// quantizer's arithmetic (outer scale amax / 2688, E4M3 block scales, E2M1
// codes, element 2i in the low nibble).
//
// Layout: W waves own one row (W = 1 for f <= 2048, else 4); lane l of the
// row's 64W lanes holds elements [4(l + 64W t), +4) for t < T, so every load
// and store instruction of a wave is contiguous, and one 16-element block is
// held by an aligned quad of lanes (block amax by two DPP quad permutes).
#include "swiglu_core.h"

namespace nvfp4 {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_stream_f4(const float4* p) {
  f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// max over the aligned quad of lanes
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp_mov<0xB1>(v));  // quad_perm [1,0,3,2]
  v = max(v, dpp_mov<0x4E>(v));  // quad_perm [2,3,0,1]
  return v;
}

template <int W, int T>
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(
    const float* __restrict__ gu, int64_t rows, int64_t f, uint16_t* __restrict__ h_out,
    float* __restrict__ amax_out, uint8_t* __restrict__ q, uint8_t* __restrict__ sb,
    float* __restrict__ s) {
  constexpr int RPB = 4 / W;  // rows per block and iteration
  constexpr int LANES = 64 * W;
  __shared__ uint32_t red[2][4];
  const int wave = threadIdx.x >> 6;
  const int sub = wave / W;
  const int lw = (wave % W) * 64 + (threadIdx.x & 63);
  const bool quantize = s != nullptr;
  int it = 0;
  for (int64_t row0 = (int64_t)blockIdx.x * RPB; row0 < rows;
       row0 += (int64_t)gridDim.x * RPB, ++it) {
    const int64_t row = row0 + sub;
    const bool row_ok = row < rows;  // uniform per wave (always true for W = 4)
    const float4* g4 = reinterpret_cast<const float4*>(gu + (row_ok ? row : 0) * 2 * f);
    const float4* u4 = reinterpret_cast<const float4*>(gu + (row_ok ? row : 0) * 2 * f + f);
    float4 gv[T], uv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t e0 = 4 * (int64_t)(lw + LANES * t);
      if (row_ok && e0 < f) {
        gv[t] = ld_stream_f4(g4 + e0 / 4);
        uv[t] = ld_stream_f4(u4 + e0 / 4);
      } else {
        gv[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        uv[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    uint32_t hb[T][2];
    uint32_t bmax[T];
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint32_t b0 = swiglu_bf16(gv[t].x, uv[t].x), b1 = swiglu_bf16(gv[t].y, uv[t].y);
      const uint32_t b2 = swiglu_bf16(gv[t].z, uv[t].z), b3 = swiglu_bf16(gv[t].w, uv[t].w);
      hb[t][0] = b0 | (b1 << 16);
      hb[t][1] = b2 | (b3 << 16);
      const uint32_t lm = max(max(b0 & 0x7FFFu, b1 & 0x7FFFu), max(b2 & 0x7FFFu, b3 & 0x7FFFu));
      bmax[t] = quad_max_u32(lm);
      m = max(m, bmax[t]);
    }
    m = group_max_u32<64>(m);
    if (W > 1) {
      if ((threadIdx.x & 63) == 0) red[it & 1][wave] = m;
      __syncthreads();
      m = max(max(red[it & 1][0], red[it & 1][1]), max(red[it & 1][2], red[it & 1][3]));
    }
    if (!row_ok) continue;
    const float amax = __uint_as_float(m << 16);
    const RowScale rs = row_scale(amax);
    if (lw == 0) {
      if (amax_out) amax_out[row] = amax;
      if (quantize) s[row] = rs.S;
    }
    // A block is a quad of lanes, all holding its amax.  Lane d of each quad
    // derives the scales of slots d, d + 4, ... and quad broadcasts hand them
    // to the other three lanes (every lane runs this, so the DPP sources are
    // live; slots past f carry amax 0 and are never stored).
    uint32_t code_t[T];
    float inv_t[T];
    if (quantize) {
      const int qd = lw & 3;
#pragma unroll
      for (int t0 = 0; t0 < T; t0 += 4) {
        uint32_t a = bmax[t0];
#pragma unroll
        for (int d = 1; d < 4; ++d)
          if (t0 + d < T) a = (qd == d) ? bmax[t0 + d] : a;
        uint32_t c;
        float v;
        block_scale(a, rs, c, v);
        const uint32_t vb = __float_as_uint(v);
        code_t[t0] = dpp_mov<0x00>(c);
        inv_t[t0] = __uint_as_float(dpp_mov<0x00>(vb));
        if (t0 + 1 < T) {
          code_t[t0 + 1] = dpp_mov<0x55>(c);
          inv_t[t0 + 1] = __uint_as_float(dpp_mov<0x55>(vb));
        }
        if (t0 + 2 < T) {
          code_t[t0 + 2] = dpp_mov<0xAA>(c);
          inv_t[t0 + 2] = __uint_as_float(dpp_mov<0xAA>(vb));
        }
        if (t0 + 3 < T) {
          code_t[t0 + 3] = dpp_mov<0xFF>(c);
          inv_t[t0 + 3] = __uint_as_float(dpp_mov<0xFF>(vb));
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t e0 = 4 * (int64_t)(lw + LANES * t);
      if (e0 >= f) continue;
      if (h_out) {  // streaming stores: H is not read again here
        uint32_t* hp = reinterpret_cast<uint32_t*>(h_out + row * f + e0);
        __builtin_nontemporal_store(hb[t][0], hp);
        __builtin_nontemporal_store(hb[t][1], hp + 1);
      }
      if (!quantize) continue;
      const uint32_t code = code_t[t];
      const float inv = inv_t[t];
      float r[4] = {__uint_as_float(hb[t][0] << 16), __uint_as_float(hb[t][0] & 0xFFFF0000u),
                    __uint_as_float(hb[t][1] << 16), __uint_as_float(hb[t][1] & 0xFFFF0000u)};
      if (__builtin_expect(__builtin_isinf(inv), 0)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (r[i] == 0.0f) ? r[i] : r[i] * inv;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] *= inv;
      }
      uint32_t c = e2m1_encode2<0>(0u, r[0], r[1]);
      c = e2m1_encode2<1>(c, r[2], r[3]);
      reinterpret_cast<uint16_t*>(q + row * (f / 2))[e0 / 4] = (uint16_t)c;
      if ((lw & 3) == 0) sb[row * (f / 16) + e0 / 16] = (uint8_t)code;
    }
  }
}

typedef void (*SwigluKernel)(const float*, int64_t, int64_t, uint16_t*, float*, uint8_t*,
                             uint8_t*, float*);

static SwigluKernel pick_swiglu(int64_t f, int& waves_per_row) {
  if (f <= 2048) {
    waves_per_row = 1;
    switch (f <= 0 ? 1 : (int)((f + 255) / 256)) {
      case 1: return swiglu_quantize_kernel<1, 1>;
      case 2: return swiglu_quantize_kernel<1, 2>;
      case 3: return swiglu_quantize_kernel<1, 3>;
      case 4: return swiglu_quantize_kernel<1, 4>;
      case 5: return swiglu_quantize_kernel<1, 5>;
      case 6: return swiglu_quantize_kernel<1, 6>;
      case 7: return swiglu_quantize_kernel<1, 7>;
      default: return swiglu_quantize_kernel<1, 8>;
    }
  }
  waves_per_row = 4;
  switch ((int)((f + 1023) / 1024)) {
    case 3: return swiglu_quantize_kernel<4, 3>;
    case 4: return swiglu_quantize_kernel<4, 4>;
    case 5: return swiglu_quantize_kernel<4, 5>;
    case 6: return swiglu_quantize_kernel<4, 6>;
    case 7: return swiglu_quantize_kernel<4, 7>;
    case 8: return swiglu_quantize_kernel<4, 8>;
    case 9: return swiglu_quantize_kernel<4, 9>;
    case 10: return swiglu_quantize_kernel<4, 10>;
    case 11: return swiglu_quantize_kernel<4, 11>;
    case 12: return swiglu_quantize_kernel<4, 12>;
    default: return nullptr;
  }
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_swiglu_quantize_rows(const float* gate_up, int64_t rows, int64_t f,
                                          uint16_t* h_out, float* amax_out, uint8_t* q,
                                          uint8_t* sb, float* s, void* stream) {
  if (rows < 0 || f < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (f % 16 != 0 || f > 12288) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (rows == 0) return NVFP4_SUCCESS;
  const bool quantize = s != nullptr;
  if (!quantize && (q || sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (quantize && f > 0 && !(q && sb)) return NVFP4_ERROR_INVALID_VALUE;
  if (!quantize && !h_out && !amax_out) return NVFP4_ERROR_INVALID_VALUE;
  if (f > 0 && !gate_up) return NVFP4_ERROR_INVALID_VALUE;
  if (rows > ((int64_t)1 << 36)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(gate_up, 16) || !aligned(h_out, 16) || !aligned(q, 16) || !aligned(s, 4) ||
      !aligned(amax_out, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.f32_finite(gate_up, rows * 2 * f);
    if ((st = chk.result())) return st;
  }
#endif
  int wpr = 1;
  nvfp4::SwigluKernel kern = nvfp4::pick_swiglu(f, wpr);
  if (!kern) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  const int64_t rpb = 4 / wpr;
  const int64_t need = (rows + rpb - 1) / rpb;
  // enough blocks for one row group per wave at the shapes of interest: with
  // no prefetch inside a wave, oversubscription is what overlaps one wave's
  // loads with another's arithmetic
  const int64_t cap = (int64_t)nvfp4host::num_cus() * 32;
  dim3 grid((unsigned)(need < cap ? need : cap));
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, (hipStream_t)stream, gate_up, rows, f, h_out,
                     amax_out, q, sb, s);
  return nvfp4host::launch_status();
}
