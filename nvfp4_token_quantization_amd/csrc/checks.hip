// checks.hip -- device-side precondition checks of the checked build
// (libnvfp4_checked.so, compiled with NVFP4_CHECKED=1).
//
// The product library leaves device-side precondition violations undefined
// (non-finite inputs give unspecified codes, bad offsets are clamped so they
// cannot fault).  The checked build runs, before an entry point's first
// launch and on its stream, small validation kernels over the arguments in
// device memory:
//  - bf16 / fp32 inputs finite (a supplied amax also >= 0);
//  - E4M3 block-scale codes not NaN (0x7F / 0xFF), E8M0 codes not 0xFF;
//  - per-expert offsets non-decreasing (values outside [0, m_total] are
//    clamped by the grouped GEMMs, which is defined).
// Each kernel ORs its bit into a device flag (one atomic per wave with a
// violation); the host zeroes the flag with a kernel, waits for the stream
// and reads the flag back, and the entry point returns
// NVFP4_ERROR_PRECONDITION without launching anything else.  A mutex
// serializes checked calls, since they share the flag.
#include <mutex>

#include "nvfp4_internal.h"

namespace nvfp4check {

__device__ unsigned int check_flag;

namespace {

__device__ __forceinline__ void report(bool bad, unsigned int bit) {
  const unsigned long long b = __ballot(bad);
  if (b && (threadIdx.x & 63) == (unsigned)__builtin_ctzll(b)) atomicOr(&check_flag, bit);
}

__global__ __launch_bounds__(64) void zero_flag_kernel() {
  if (threadIdx.x == 0) check_flag = 0u;
}

__global__ __launch_bounds__(256) void bf16_finite_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                          unsigned int bit) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= (x[i] & 0x7F80u) == 0x7F80u;
  report(bad, bit);
}

__global__ __launch_bounds__(256) void f32_finite_kernel(const float* __restrict__ x, int64_t n,
                                                         bool nonneg, unsigned int bit) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = x[i];
    bad |= !__builtin_isfinite(v) || (nonneg && v < 0.0f);
  }
  report(bad, bit);
}

// E4M3 (mask 0x7F) or E8M0 (mask 0xFF) codes equal to their NaN pattern
__global__ __launch_bounds__(256) void nan_codes_kernel(const uint8_t* __restrict__ c, int64_t n,
                                                        uint32_t mask, unsigned int bit) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= (c[i] & mask) == mask;
  report(bad, bit);
}

__global__ __launch_bounds__(256) void offsets_kernel(const int32_t* __restrict__ off, int64_t groups,
                                                      unsigned int bit) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < groups; i += (int64_t)gridDim.x * 256)
    bad |= off[i + 1] < off[i];
  report(bad, bit);
}

dim3 grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return dim3((unsigned)(b < 1 ? 1 : (b > 1024 ? 1024 : b)));
}

std::mutex check_mutex;

}  // namespace

Checks::Checks(hipStream_t s) : stream(s) {
  check_mutex.lock();
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(64), 0, stream);
}

Checks::~Checks() {
  if (!done) check_mutex.unlock();
}

void Checks::bf16_finite(const uint16_t* x, int64_t n) {
  if (x && n > 0) hipLaunchKernelGGL(bf16_finite_kernel, grid_for(n), dim3(256), 0, stream, x, n, 1u);
}

void Checks::f32_finite(const float* x, int64_t n, bool nonneg) {
  if (x && n > 0) hipLaunchKernelGGL(f32_finite_kernel, grid_for(n), dim3(256), 0, stream, x, n, nonneg, 2u);
}

void Checks::e4m3_codes(const uint8_t* c, int64_t n) {
  if (c && n > 0) hipLaunchKernelGGL(nan_codes_kernel, grid_for(n), dim3(256), 0, stream, c, n, 0x7Fu, 4u);
}

void Checks::e8m0_codes(const uint8_t* c, int64_t n) {
  if (c && n > 0) hipLaunchKernelGGL(nan_codes_kernel, grid_for(n), dim3(256), 0, stream, c, n, 0xFFu, 4u);
}

void Checks::offsets(const int32_t* off, int64_t groups) {
  if (off && groups > 0) hipLaunchKernelGGL(offsets_kernel, grid_for(groups), dim3(256), 0, stream, off, groups, 8u);
}

int Checks::result() {
  unsigned int h = 0u;
  int st = NVFP4_SUCCESS;
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyFromSymbolAsync(&h, HIP_SYMBOL(check_flag), sizeof(h), 0, hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    st = NVFP4_ERROR_LAUNCH;
  else if (h)
    st = NVFP4_ERROR_PRECONDITION;
  done = true;
  check_mutex.unlock();
  return st;
}

}  // namespace nvfp4check
