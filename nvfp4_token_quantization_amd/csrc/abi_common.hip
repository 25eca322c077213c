// abi_common.hip -- version and status strings of libnvfp4.so.
#include "nvfp4_internal.h"

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
    case NVFP4_ERROR_PRECONDITION:
      return "device-side precondition violated (non-finite input or scale, NaN scale code, decreasing offsets)";
    default: return "unknown status";
  }
}

}  // extern "C"
