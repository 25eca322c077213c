// abi_common.hip -- version, status strings, architecture check and the
// codec self-test hooks of libnvfp4.so.
#include <string.h>

#include "nvfp4_internal.h"

namespace nvfp4host {

int check_arch() {
  // 0 = unknown, 1 = gfx950, 2 = other; one slot per device ordinal
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERROR_ARCH;
  if (dev < 0 || dev >= 64) return NVFP4_ERROR_ARCH;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
  if (v == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return NVFP4_ERROR_ARCH;
    v = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELEASE);
  }
  return v == 1 ? NVFP4_SUCCESS : NVFP4_ERROR_ARCH;
}

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELEASE);
  }
  return v;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH;
}

}  // namespace nvfp4host

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

}  // namespace nvfp4

extern "C" {

int nvfp4_version(void) { return 100; /* 0.1.0 */ }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_SUCCESS: return "success";
    case NVFP4_ERROR_INVALID_VALUE: return "invalid value (null pointer, negative size or zero groups)";
    case NVFP4_ERROR_UNSUPPORTED_SHAPE: return "unsupported shape (k % 16 != 0 or a size past a stated limit)";
    case NVFP4_ERROR_MISALIGNED: return "misaligned pointer";
    case NVFP4_ERROR_LAUNCH: return "kernel launch failed";
    case NVFP4_ERROR_ARCH: return "current device is not gfx950";
    default: return "unknown status";
  }
}

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

}  // extern "C"
