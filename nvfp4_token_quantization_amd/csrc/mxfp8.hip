// mxfp8.hip -- MXFP8 quantization (gfx950): 32 consecutive values along K
// share one E8M0 power-of-two scale, values are E4M3.
//
// The Miles page (section MXFP8格式背景) describes the format and its scale
// rule: the decoded scale is rounded up so the block maximum is never
// clipped.  Here 2^e is the smallest power of two with a_b / 2^e <= 448,
// computed exactly from the bf16 bits of the block amax a_b = m 2^E
// (1 <= m < 2): e = E - 8 when m <= 1.75 (448 = 1.75 * 2^8), else E - 7.
// Code e + 127 is clamped to [0, 254]; zero and subnormal-amax blocks take 0.
// Elements: x * 2^-e is exact (a power-of-two scaling; results below 2^-126
// are far under E4M3's smallest step and round to zero either way) and
// gfx950's pack-convert rounds it to E4M3 (nearest even, sign kept).
//
// Layout: the [rows, k] tensor is a flat run of 16-byte chunks (8 elements);
// lane l of a wave takes chunks base + l + 64 u (u < U), so every load
// instruction reads 1 KB contiguous.  A 32-element block is an aligned quad
// of lanes: two DPP steps give all four lanes the block amax and its scale,
// each lane converts its 8 elements into 8 bytes (non-temporal stores: the
// codes are not read again here) and the quad's first lane stores the scale.
#include "mxfp8_codec.h"

namespace nvfp4 {

template <typename IDX, int U>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t* __restrict__ x,
                                                             IDX nchunks, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const IDX step = (IDX)64 * U;
  const IDX stride = (IDX)gridDim.x * 4 * step;
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  // wave-uniform loop; nchunks is a multiple of 4 and base of 64, so a quad
  // is either wholly inside the tensor or wholly past its end
  for (IDX base = ((IDX)blockIdx.x * 4 + (threadIdx.x >> 6)) * step; base < nchunks;
       base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const IDX c = base + lane + 64 * u;
      v[u] = c < nchunks ? ld_stream(x4 + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const IDX c = base + lane + 64 * u;
      uint32_t a = half_amax_bits(v[u]);
      a = max(a, dpp_mov<0xB1>(a));  // quad_perm [1,0,3,2]
      a = max(a, dpp_mov<0x4E>(a));  // quad_perm [2,3,0,1]
      const uint32_t code = mx_scale_code(a);
      const float inv = __uint_as_float((254u - code) << 23);  // 2^-(code - 127)
      if (c < nchunks) {
        uint32_t* qo = reinterpret_cast<uint32_t*>(q) + 2 * (int64_t)c;
        __builtin_nontemporal_store(fp8_encode4(v[u].x, v[u].y, inv), qo);
        __builtin_nontemporal_store(fp8_encode4(v[u].z, v[u].w, inv), qo + 1);
        if ((lane & 3) == 0) sc[c >> 2] = (uint8_t)code;
      }
    }
  }
}

}  // namespace nvfp4

using nvfp4host::aligned;

extern "C" int nvfp4_mxfp8_quantize_rows(const uint16_t* x_bf16, int64_t rows, int64_t k,
                                         uint8_t* q, uint8_t* sc, void* stream) {
  if (rows < 0 || k < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 32 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (rows == 0 || k == 0) return NVFP4_SUCCESS;
  if (!x_bf16 || !q || !sc) return NVFP4_ERROR_INVALID_VALUE;
  if (rows > ((int64_t)1 << 36) || k > ((int64_t)1 << 30)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
#if NVFP4_CHECKED
  {
    nvfp4check::Checks chk((hipStream_t)stream);
    chk.bf16_finite(x_bf16, rows * k);
    if ((st = chk.result())) return st;
  }
#endif
  const int64_t nchunks = rows * (k / 8);  // 16-byte chunks, 4 per block
  constexpr int U = 4;
  const int64_t need = (nchunks + 256 * U - 1) / (256 * U);
  const int64_t cap = (int64_t)nvfp4host::num_cus() * 32;
  dim3 grid((unsigned)(need < cap ? need : cap));
  hipStream_t str = (hipStream_t)stream;
  if (nchunks + (int64_t)grid.x * 256 * U < ((int64_t)1 << 31))
    hipLaunchKernelGGL((nvfp4::mxfp8_quantize_kernel<uint32_t, U>), grid, dim3(256), 0, str, x_bf16,
                       (uint32_t)nchunks, q, sc);
  else
    hipLaunchKernelGGL((nvfp4::mxfp8_quantize_kernel<uint64_t, U>), grid, dim3(256), 0, str, x_bf16,
                       (uint64_t)nchunks, q, sc);
  return nvfp4host::launch_status();
}
