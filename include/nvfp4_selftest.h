/*
 * nvfp4_selftest.h -- codec self-test hooks of libnvfp4_selftest.so.
 *
 * Test-only: these calls are not part of the libnvfp4.so boundary.  They run
 * the quantizers' device rounding functions on arbitrary fp32 inputs so that
 * tests can compare them with the reference codec on every bit pattern.
 * Status codes are those of nvfp4.h.
 */
#ifndef NVFP4_SELFTEST_H
#define NVFP4_SELFTEST_H

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Self-test hooks: apply the device rounding functions the quantizer uses to
 * arbitrary fp32 inputs, so tests can sweep every bit pattern; and run the
 * one-pass weight quantizer on shapes and time limits of a test's choosing.
 *   nvfp4_debug_encode_e2m1: code[i] = 4-bit E2M1 code (sign | RNE_SAT
 *     magnitude) of v[i]; +-inf saturate; NaN inputs give unspecified codes.
 *   nvfp4_debug_encode_e4m3: code[i] = RNE_SAT E4M3 code of v[i] >= 0
 *     (+inf saturates to 0x7E); negative or NaN inputs give unspecified codes.
 * v [n] f32 device, code [n] u8 device.  Errors as above.
 */
int nvfp4_debug_encode_e2m1(const float* v, int64_t n, uint8_t* code, void* stream);
/* nvfp4_debug_encode_fp8: code[i] = E4M3 code (sign | RNE_SAT magnitude) of
 * v[i] through the pack-convert the MXFP8 quantizer uses; only |v| <= 448
 * and +-0 are specified (the quantizer never converts larger values). */
int nvfp4_debug_encode_fp8(const float* v, int64_t n, uint8_t* code, void* stream);
int nvfp4_debug_encode_e4m3(const float* v, int64_t n, uint8_t* code, void* stream);
/* nvfp4_debug_block_scale: the quantizer's per-block scale step (Miles page,
 * section 速读: E4M3 block scale under the FP32 outer scale) on arbitrary
 * inputs.  For each i, with S = fl32(amax[i] / 2688) and a = the bf16 value
 * of block_amax[i] (sign bit ignored):
 *   code[i] = RNE_SAT_E4M3(fl32(a / fl32(6 S)))   (0 when S == 0)
 *   inv[i]  = fl32(1 / fl32(S * e4m3(code[i])))    (0 when that product is 0)
 * block_amax [n] u16 (bf16 bits), amax [n] f32, code [n] u8, inv [n] f32,
 * all device memory.  amax[i] must be finite and >= 0.  Errors as above. */
int nvfp4_debug_block_scale(const uint16_t* block_amax, const float* amax, int64_t n,
                            uint8_t* code, float* inv, void* stream);
/* nvfp4_debug_quantize_weight_onepass: nvfp4_quantize_weight (amax_in NULL)
 * forced onto its one-pass kernel, at any group size, with each workgroup's
 * wait for its team bounded by limit_ms milliseconds (0: a workgroup that
 * does not find every member arrived at once takes the group amax by reading
 * the whole group itself).  Arguments and outputs as nvfp4_quantize_weight;
 * amax_out and s must not overlap.  UNSUPPORTED_SHAPE when the one-pass
 * kernel cannot hold a group (the library then uses two passes). */
int nvfp4_debug_quantize_weight_onepass(const uint16_t* w_bf16, int64_t groups, int64_t rows_per_group,
                                        int64_t k, float* amax_out, uint8_t* q, uint8_t* sb, float* s,
                                        double limit_ms, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_SELFTEST_H */
