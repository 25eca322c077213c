// host_util.hip -- host-side helpers shared by libnvfp4.so and the codec
// self-test library: the gfx950 check, CU count and wall-clock rate per
// device (cached), and the launch status.
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

int64_t wall_clock_khz() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100000;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess || v <= 0)
      v = 100000;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELEASE);
  }
  return v;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? NVFP4_SUCCESS : NVFP4_ERROR_LAUNCH;
}

}  // namespace nvfp4host
