// selftest.hip -- libnvfp4_selftest.so: self-test hooks that apply the device
// rounding functions of the quantizers to arbitrary fp32 inputs, so tests can
// sweep every bit pattern, and run the one-pass weight quantizer on any group
// size with a chosen bound on its wait.  Test-only: not part of libnvfp4.so
// or of its header; declared in include/nvfp4_selftest.h.
#include "mxfp8_codec.h"
#include "weight_onepass.h"
#include "nvfp4_selftest.h"

namespace nvfp4 {

__global__ __launch_bounds__(256) void debug_e2m1_kernel(const float* __restrict__ v, int64_t n,
                                                         uint8_t* __restrict__ code) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) code[i] = (uint8_t)(e2m1_encode2<0>(0u, v[i], 0.0f) & 15u);
}

__global__ __launch_bounds__(256) void debug_e4m3_kernel(const float* __restrict__ v, int64_t n,
                                                         uint8_t* __restrict__ code) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) code[i] = (uint8_t)e4m3_encode(v[i]);
}

__global__ __launch_bounds__(256) void debug_block_scale_kernel(const uint16_t* __restrict__ bmax,
                                                                const float* __restrict__ amax,
                                                                int64_t n,
                                                                uint8_t* __restrict__ code,
                                                                float* __restrict__ inv) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  uint32_t c;
  float r;
  block_scale(bmax[i] & 0x7FFFu, row_scale(amax[i]), c, r);
  code[i] = (uint8_t)c;
  inv[i] = r;
}

__global__ __launch_bounds__(256) void debug_fp8_kernel(const float* __restrict__ v, int64_t n,
                                                        uint8_t* __restrict__ code) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    code[i] = (uint8_t)(fp8_encode2<false>(0u, v[i], 0.0f) & 0xFFu);
}

}  // namespace nvfp4

extern "C" {

static int debug_launch(int which, const float* v, int64_t n, uint8_t* code, void* stream) {
  if (n < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (n == 0) return NVFP4_SUCCESS;
  if (!v || !code) return NVFP4_ERROR_INVALID_VALUE;
  if (!nvfp4host::aligned(v, 4)) return NVFP4_ERROR_MISALIGNED;
  if (n > ((int64_t)1 << 40)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  int st = nvfp4host::check_arch();
  if (st) return st;
  dim3 grid((unsigned)((n + 255) / 256));
  if (which == 0)
    hipLaunchKernelGGL(nvfp4::debug_e2m1_kernel, grid, dim3(256), 0, (hipStream_t)stream, v, n, code);
  else
    hipLaunchKernelGGL(nvfp4::debug_e4m3_kernel, grid, dim3(256), 0, (hipStream_t)stream, v, n, code);
  return nvfp4host::launch_status();
}

int nvfp4_debug_encode_e2m1(const float* v, int64_t n, uint8_t* code, void* stream) {
  return debug_launch(0, v, n, code, stream);
}

int nvfp4_debug_encode_e4m3(const float* v, int64_t n, uint8_t* code, void* stream) {
  return debug_launch(1, v, n, code, stream);
}

int nvfp4_debug_block_scale(const uint16_t* block_amax, const float* amax, int64_t n,
                            uint8_t* code, float* inv, void* stream) {
  if (n < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (n == 0) return NVFP4_SUCCESS;
  if (!block_amax || !amax || !code || !inv) return NVFP4_ERROR_INVALID_VALUE;
  if (!nvfp4host::aligned(block_amax, 2) || !nvfp4host::aligned(amax, 4) ||
      !nvfp4host::aligned(inv, 4))
    return NVFP4_ERROR_MISALIGNED;
  if (n > ((int64_t)1 << 40)) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  int st = nvfp4host::check_arch();
  if (st) return st;
  dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(nvfp4::debug_block_scale_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     block_amax, amax, n, code, inv);
  return nvfp4host::launch_status();
}

int nvfp4_debug_encode_fp8(const float* v, int64_t n, uint8_t* code, void* stream) {
  if (n < 0) return NVFP4_ERROR_INVALID_VALUE;
  if (n == 0) return NVFP4_SUCCESS;
  if (!v || !code) return NVFP4_ERROR_INVALID_VALUE;
  if (!nvfp4host::aligned(v, 4)) return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  const int64_t need = (n + 255) / 256;
  dim3 grid((unsigned)(need < 4096 ? need : 4096));
  hipLaunchKernelGGL(nvfp4::debug_fp8_kernel, grid, dim3(256), 0, (hipStream_t)stream, v, n, code);
  return nvfp4host::launch_status();
}

int nvfp4_debug_quantize_weight_onepass(const uint16_t* w, int64_t groups, int64_t rows_per_group,
                                        int64_t k, float* amax_out, uint8_t* q, uint8_t* sb, float* s,
                                        double limit_ms, void* stream) {
  if (groups < 1 || rows_per_group < 1 || k < 16 || !(limit_ms >= 0.0)) return NVFP4_ERROR_INVALID_VALUE;
  if (k % 16 != 0) return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!w || !amax_out || !q || !sb || !s) return NVFP4_ERROR_INVALID_VALUE;
  if (groups * rows_per_group > ((int64_t)1 << 36) || k > ((int64_t)1 << 30))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  if (!nvfp4host::aligned(w, 16) || !nvfp4host::aligned(q, 16) || !nvfp4host::aligned(s, 4) ||
      !nvfp4host::aligned(amax_out, 4))
    return NVFP4_ERROR_MISALIGNED;
  int st = nvfp4host::check_arch();
  if (st) return st;
  if (!nvfp4::launch_weight_onepass(w, groups, rows_per_group, k, amax_out, q, sb, s, limit_ms, 0, 1,
                                    (hipStream_t)stream))
    return NVFP4_ERROR_UNSUPPORTED_SHAPE;
  return nvfp4host::launch_status();
}

}  // extern "C"
