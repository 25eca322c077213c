/*
 * nvfp4.h -- C ABI of libnvfp4.so: per-token NVFP4 quantization and the
 * block-scaled W4A4 linear it feeds, for AMD Instinct MI355X (gfx950).
 *
 * NVFP4 as used here (see the pages named in each declaration):
 *   x_hat = S * s_b * e2m1(q)
 *   q   : 4-bit E2M1 code (sign, 2 exponent bits, 1 mantissa bit), two per
 *         byte, element 2i in the low nibble of byte i;
 *   s_b : one E4M3 (OCP "FN", max 448) block scale per 16 consecutive
 *         elements along the contraction axis K;
 *   S   : FP32 outer scale, per row (per token) for activations, per tensor
 *         or per expert for weights.
 *
 * Quantization contract (one result is correct; it is reproduced bit for bit):
 *   S     = fl32(amax / 2688)                         (2688 = 6 * 448)
 *   s_b   = RNE_SAT_E4M3(fl32(a_b / fl32(6 * S)))      (0 when S == 0)
 *   d     = fl32(S * s_b)
 *   code  = sign(x) | RNE_SAT_E2M1(|fl32(x * fl32(1 / d))|)
 *           (magnitude 0 when d == 0 or x == +-0)
 * RNE_SAT rounds to the nearest finite code value with ties to the even code
 * and saturates (values above the maximum and +inf give the maximum).  amax
 * is the row (or group) max of |x|; a_b is the block max of |x|.
 *
 * Layouts (all row-major, canonical, no padding or swizzling):
 *   bf16 input  [rows, k]          -> q [rows, k/2] u8, sb [rows, k/16] u8
 *   per-token S [rows] f32;  weight S [groups] f32
 *   GEMM: Y[m, n] = sum_k x_hat_A[m, k] * x_hat_B[n, k]  (both K-major,
 *   blocks along K), Y fp32 [m, n] row-major.
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller.  The library never
 *     allocates, frees or keeps them.  Inputs are read-only; outputs are
 *     overwritten; inputs and outputs must not overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls are asynchronous and never synchronize the host.  The host never
 *     reads device data (grouped GEMM offsets stay on the device).
 *   - Return value: NVFP4_SUCCESS or an error code.  Argument errors are
 *     detected before any HIP call and launch nothing.  NVFP4_ERROR_LAUNCH
 *     reports a failed launch (hipGetLastError).  NVFP4_ERROR_ARCH: the
 *     current device is not gfx950.
 *   - Alignment: tensor pointers must be 16-byte aligned (fp32 scale
 *     vectors 4-byte aligned).
 *   - GEMM sizes: besides each call's own limits, an output whose tile grid
 *     ((m_total / 128 + groups + 1) x (n / 64 + 1)) passes 2^28 tiles -- far
 *     beyond device memory -- is rejected with UNSUPPORTED_SHAPE.
 *   - Inputs must be finite; non-finite bf16 inputs give unspecified codes
 *     (no fault).  Stateless and re-entrant; calls on one stream are ordered.
 *   - Device-side preconditions (values in device memory, which the host
 *     never reads) are undefined when violated, never a fault: non-finite
 *     bf16 / f32 inputs, supplied amax or scales (a supplied amax also < 0),
 *     NaN E4M3 block-scale codes (0x7F, 0xFF) or E8M0 codes (0xFF), and
 *     offsets that decrease.  The checked build, libnvfp4_checked.so, made
 *     from the same sources with NVFP4_CHECKED=1, validates them on the
 *     call's stream before launching anything else, waits for the stream
 *     and returns NVFP4_ERROR_PRECONDITION on a violation (outputs then
 *     untouched).  It synchronizes the host and serializes its calls, so it
 *     is a debugging aid that cannot be captured in a graph; the product
 *     library never checks these values and never returns that status.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_SUCCESS 0
#define NVFP4_ERROR_INVALID_VALUE 1     /* null pointer, negative size, zero groups */
#define NVFP4_ERROR_UNSUPPORTED_SHAPE 2 /* k % 16 != 0, or a size past a stated limit */
#define NVFP4_ERROR_MISALIGNED 3        /* pointer alignment below the stated minimum */
#define NVFP4_ERROR_LAUNCH 4            /* kernel launch failed */
#define NVFP4_ERROR_ARCH 5              /* current device is not gfx950 */
#define NVFP4_ERROR_PRECONDITION 6      /* checked build only: see below */

/* Library version, major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

/* Static string naming a status code (never NULL). */
const char* nvfp4_status_string(int status);

/*
 * Per-token NVFP4 activation quantization.
 *
 * Defined by: "Towards Blackwell-Native 8-bit and 4-bit RL: End-to-End MXFP8
 * and NVFP4 RL in Miles", section 速读 (X ~ s_token * s_block * X_FP4, 16 E2M1
 * values per E4M3 block scale) and section 单Token缩放的在线计算实现 (the FP32
 * per-token scale is computed online inside the quantize call, which returns
 * packed FP4, E4M3 block scales and the per-token scale together); decode
 * formula on "TRIAGE: Direction-Aware Mismatch Stabilization of Native NVFP4
 * Reinforcement Learning", section 前置知识.  Amax reuse ("miniTE报告", section
 * Transformer Engine路径优化) is the amax_in argument.
 *
 *   x_bf16  [rows, k] bf16 bit patterns, k % 16 == 0 (k may be 0)
 *   amax_in NULL: amax = max_k |x[r, k]| computed here.
 *           else [rows] f32: amax of row r is amax_in[r] (the producer's
 *           statistic; bits are a function of (x, amax_in)).
 *   q       [rows, k/2] u8 out;  sb [rows, k/16] u8 out;  s [rows] f32 out (S)
 * Each row's output depends only on that row (batch invariant).
 * Errors: INVALID_VALUE (rows or k < 0; null x, q, sb or s when there is work),
 * UNSUPPORTED_SHAPE (k % 16 != 0), MISALIGNED, ARCH, LAUNCH.
 */
int nvfp4_quantize_rows(const uint16_t* x_bf16, int64_t rows, int64_t k, const float* amax_in,
                        uint8_t* q, uint8_t* sb, float* s, void* stream);

/*
 * Weight NVFP4 quantization with a per-tensor or per-expert FP32 outer scale.
 *
 * Defined by: "miniTE报告" section NVFP4格式、两级缩放与转换误差 (the outer
 * scale may be per tensor, per expert or per row) and the Miles page, section
 * 并行度与张量转换的一致性契约 (fused gate/up weights share one FP32 scale:
 * pass the fused [2I, H] expert weight as one group); weights use 1D 1x16
 * blocks along K (Miles page, recipe under 补充细节, 2D quantization disabled).
 *
 *   w_bf16   [groups, rows_per_group, k] bf16 bits, k % 16 == 0
 *   amax_in  NULL: amax[g] = max |w[g]| reduced here (into amax_out).
 *            else [groups] f32 used as the group amax.
 *   amax_out [groups] f32 out: the group amax (required when amax_in is
 *            NULL, where it also serves as the reduction target; optional
 *            otherwise, then a copy of amax_in).
 *   q [groups*rows_per_group, k/2] u8 out; sb [groups*rows_per_group, k/16] u8
 *   out; s [groups] f32 out (S per group).
 * Each row is encoded exactly as nvfp4_quantize_rows would encode it with
 * amax_in set to its group's amax.  Errors as for nvfp4_quantize_rows, plus
 * INVALID_VALUE for groups < 1, a missing amax_out, or amax_out and s
 * overlapping.
 * When the amax is computed here and there are at least 8 groups of at
 * least 512 KiB of bf16, the weight is read once: while the call runs,
 * amax_out[g], s[g] and the first 256 bytes of group g's codes in q hold the
 * partial maxima and counts of the workgroups that share group g (all hold
 * their final values when the call's work completes).  amax_out, s and q
 * must not overlap each other or the other buffers.  No workspace is
 * allocated.  Work on other
 * streams may hold CUs that the call's workgroups wait for: a workgroup
 * waits at most 10 ms for its team before reading the group itself for its
 * amax, so the results are exact in every case.
 */
int nvfp4_quantize_weight(const uint16_t* w_bf16, int64_t groups, int64_t rows_per_group,
                          int64_t k, const float* amax_in, float* amax_out, uint8_t* q,
                          uint8_t* sb, float* s, void* stream);

/*
 * SwiGLU of a fused gate|up projection, fused with per-token NVFP4
 * quantization of its bf16 output (the row amax never leaves the kernel).
 *
 * Defined by: the miniTE page, section Transformer Engine路径优化 (amax reuse
 * and fusion around the grouped GEMMs), and the Miles page, section
 * 并行度与张量转换的一致性契约 (the MoE layers' gate and up projections are one
 * fused GEMM); SwiGLU is silu(gate) * up with silu(g) = g / (1 + e^-g).
 *
 *   gate_up  [rows, 2f] f32: columns [0, f) gate, [f, 2f) up of one token
 *            (the output of a GEMM against the fused [2f, K] weight).
 *            f % 16 == 0, f <= 12288.  Values and results must be finite.
 *   h_out    NULL or [rows, f] bf16 bits out: h = bf16(fl32(g * u / (1 +
 *            exp(-g)))), the quotient formed in fp64, both roundings to
 *            nearest even.
 *   amax_out NULL or [rows] f32 out: max_j |h[r, j]| (the amax to reuse).
 *   q, sb, s all NULL (produce only h and/or amax), or all given (q and sb
 *            may be NULL when f == 0): the quantization of h, bit-identical to nvfp4_quantize_rows(h, rows,
 *            f, amax_in = NULL or amax_out, q, sb, s).
 * At least one output is required.  Each row depends only on its own row.
 * Errors: INVALID_VALUE (negative sizes, a partial q/sb/s set, no output,
 * null gate_up with work), UNSUPPORTED_SHAPE (f % 16 != 0, f > 12288),
 * MISALIGNED (gate_up, h_out, q need 16 bytes; s, amax_out 4), ARCH, LAUNCH.
 */
int nvfp4_swiglu_quantize_rows(const float* gate_up, int64_t rows, int64_t f, uint16_t* h_out,
                               float* amax_out, uint8_t* q, uint8_t* sb, float* s,
                               void* stream);

/*
 * Top-k MoE routing into the contiguous per-expert layout, on the device.
 *
 * Defined by: the miniTE page, section Transformer Engine路径优化 (contiguous
 * layouts and device-side metadata feed the grouped GEMMs; tokens are
 * quantized once and gathered); each token goes to the experts with its
 * top-k router logits (softmax is monotone, so the logits decide).
 *
 *   logits      [tokens, num_experts] f32, finite (non-finite logits give an
 *               unspecified but in-range routing).
 *   experts     [tokens, topk] i32 out: the chosen experts of each token,
 *               largest logit first, the lower expert id first among equal
 *               logits (+0 equals -0).
 *   offsets     [num_experts + 1] i32 out: offsets[e] = routed rows of experts
 *               below e; offsets[num_experts] = tokens * topk.
 *   row_index   [tokens * topk] i32 out: token of each routed row; rows are
 *               ordered by expert, then by token (the layout
 *               nvfp4_grouped_gemm reads with row_index).
 *   slot_of     [tokens, topk] i32 out: routed row of each (token, choice).
 * 1 <= topk <= num_experts, num_experts <= 1024, topk <= 64,
 * tokens * topk < 2^31.  The result is deterministic (no atomics).  The
 * layout passes run one workgroup per expert, each reading all tokens * topk
 * choices (from L2 at MoE batch sizes).
 * Errors: INVALID_VALUE (negative tokens, topk < 1 or > num_experts, null
 * pointers with work; offsets is always written), UNSUPPORTED_SHAPE
 * (num_experts > 1024, topk > 64, too many rows), MISALIGNED (4 bytes), ARCH,
 * LAUNCH.
 */
int nvfp4_moe_route(const float* logits, int64_t tokens, int64_t num_experts, int64_t topk,
                    int32_t* experts, int32_t* offsets, int32_t* row_index, int32_t* slot_of,
                    void* stream);

/*
 * NVFP4 -> bf16 dequantization, for backward GEMMs that consume the
 * dequantized forward operands.
 *
 * Defined by: the Miles page, section 反量化反向模式 (the dequantized backward
 * runs its GEMMs in BF16 on the BF16 dequantization of the exact
 * low-precision forward operands) and the decode x_hat = S * s_b * e2m1(q)
 * of the TRIAGE page, section 前置知识.
 *
 *   q [rows, k/2] u8, sb [rows, k/16] u8 (E4M3 codes 0..0x7E; the sign bit
 *   is ignored, NaN codes give unspecified values), s [ceil(rows /
 *   rows_per_scale)] f32: row r uses s[r / rows_per_scale] (1 for per-token
 *   scales, rows_per_group for per-tensor / per-expert weights).
 *   x_bf16 [rows, k] bf16 out: bf16(S * s_b * e2m1(q)), the product exact
 *   and rounded once to nearest even; -0 codes give -0.
 * Errors: INVALID_VALUE (negative sizes, rows_per_scale < 1, null pointers
 * with work), UNSUPPORTED_SHAPE (k % 16 != 0), MISALIGNED (q and x_bf16 16
 * bytes, s 4), ARCH, LAUNCH.
 */
int nvfp4_dequantize_rows(const uint8_t* q, const uint8_t* sb, const float* s, int64_t rows,
                          int64_t k, int64_t rows_per_scale, uint16_t* x_bf16, void* stream);

/*
 * MXFP8 quantization: 32 consecutive values along k share one E8M0
 * power-of-two scale; the values are E4M3.
 *
 * Defined by: the Miles page, section MXFP8格式背景 (1D blocks of 32 E4M3
 * values with a local E8M0 scale, the decoded scale rounded up so the block
 * maximum is not clipped).  Scale 2^e = the smallest power of two with
 * a_b / 2^e <= 448 (a_b = block amax); code e + 127, clamped to [0, 254];
 * zero blocks take code 0.  Element code = RNE_SAT_E4M3(|x| / 2^e) with the
 * sign of x in bit 7.
 *
 *   x_bf16 [rows, k] bf16 bits, k % 32 == 0, finite.
 *   q  [rows, k] u8 out (E4M3 codes);  sc [rows, k/32] u8 out (E8M0 codes).
 * Errors: INVALID_VALUE, UNSUPPORTED_SHAPE (k % 32 != 0), MISALIGNED (x and
 * q 16 bytes), ARCH, LAUNCH.
 */
int nvfp4_mxfp8_quantize_rows(const uint16_t* x_bf16, int64_t rows, int64_t k, uint8_t* q,
                              uint8_t* sc, void* stream);

/*
 * MXFP8 GEMM: Y = deq(A) . deq(B)^T with deq = 2^(sc - 127) * e4m3(q) per
 * 32-block along k, fp32 accumulation and output.  Every element is decoded
 * exactly to bf16 (an E4M3 value times a power of two) and the products,
 * exact in fp32, are summed on the bf16 MFMA.
 *
 * Defined by: the Miles page, section MXFP8格式背景 (the format), and section
 * 配方1：端到端MXFP8 RL的设计 (forward, rollout and both gradient GEMMs run
 * in MXFP8); blocks follow the contraction axis for both operands (section
 * 案例研究：MXFP8 MLA投影张量).
 *
 *   a_q [m, k] u8 E4M3 codes, a_sc [m, k/32] u8 E8M0 codes (as written by
 *   nvfp4_mxfp8_quantize_rows); b_q [n, k], b_sc [n, k/32]; y [m, n] f32 out.
 *   k % 32 == 0 (k % 128 == 0 with 4-byte aligned scale rows takes the fast
 *   path).  Scale code 0xFF (NaN in E8M0; the quantizer never writes it)
 *   gives unspecified outputs.
 * Accuracy as nvfp4_gemm for blocks whose decoded values are bf16 numbers:
 * every scale code from 10 to 246, which the quantizer writes for every
 * block whose largest magnitude is at least 2^-109.
 * Errors: INVALID_VALUE, UNSUPPORTED_SHAPE (k % 32 != 0), MISALIGNED (a_q,
 * b_q, y 16 bytes), ARCH, LAUNCH.
 */
int nvfp4_mxfp8_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t m, const uint8_t* b_q,
                     const uint8_t* b_sc, int64_t n, int64_t k, float* y, void* stream);

/*
 * Grouped (MoE) MXFP8 GEMM over the contiguous per-expert layout: output
 * rows [offsets[g], offsets[g+1]) use expert g's weight; row_index as for
 * nvfp4_grouped_gemm (quantize each token once, gather its routed copies).
 *   a_q [a_rows, k], a_sc [a_rows, k/32]; row_index NULL or [m_total] i32;
 *   offsets [groups+1] i32 device; b_q [groups, n, k], b_sc [groups, n, k/32];
 *   y [m_total, n] f32 out (rows at or past offsets[groups] not written).
 * Accuracy as nvfp4_mxfp8_gemm.  groups <= 1024.  Errors as for
 * nvfp4_grouped_gemm (k % 32 != 0 is UNSUPPORTED_SHAPE).
 */
int nvfp4_mxfp8_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t a_rows,
                             const int32_t* row_index, int64_t m_total, const int32_t* offsets,
                             int64_t groups, const uint8_t* b_q, const uint8_t* b_sc, int64_t n,
                             int64_t k, float* y, void* stream);

/*
 * Dense block-scaled W4A4 GEMM: Y = deq(A) . deq(B)^T with the per-token
 * scale and the weight scale applied in the epilogue, Y = S_A[m] * S_B *
 * sum_k (s_bA q_A)(s_bB q_B).
 *
 * Defined by: the Miles page, section 速读 (X ~ s_token * s_block * X_FP4) and
 * 实验结果 item 10 (the per-token FP32 scale belongs in the GEMM epilogue, not
 * a separate op); blocks run along the contraction axis (Miles page, section
 * 案例研究：MXFP8 MLA投影张量).
 *
 *   A: a_q [m, k/2], a_sb [m, k/16], a_s [m] (per-token S)
 *   B: b_q [n, k/2], b_sb [n, k/16], b_s [1] (per-tensor S)
 *   y  [m, n] f32 out
 * Accuracy: the operands are decoded exactly and their products summed in
 * fp32 in an unspecified order, with at most k/16 + 2 roundings on any path
 * into an output (MFMA steps, the sum of K-split partials, the scale
 * product).  The worst case is therefore |Y - Y_exact| <= (k/16 + 2) 2^-24
 * sum_k |a_k b_k|, which is below 1e-5 sum_k |a_k b_k| for k <= 2560; above
 * that the guarantee is the (k/16 + 2) 2^-24 bound (6.1e-5 at k = 16384).
 * Tests at k = 8192 and 16384 with same-sign operands, where rounding errors
 * cannot cancel, observe at most 2e-6 sum_k |a_k b_k|.
 * Determinism: repeated calls give identical bits, and each output row
 * depends only on its own A row and B once the kernel is chosen.  m <= 64
 * with k % 256 == 0 takes the few-rows kernel, whose K-split partial sums
 * round differently from the tiled kernels taken otherwise.  So a row's last
 * bits can differ between a call with m <= 64 and one with m > 64, both
 * within the bound above.
 * Errors: INVALID_VALUE, UNSUPPORTED_SHAPE (k % 16 != 0), MISALIGNED, ARCH,
 * LAUNCH.  m, n or k == 0 are allowed (k == 0 writes zeros).
 */
int nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s, int64_t m,
               const uint8_t* b_q, const uint8_t* b_sb, const float* b_s, int64_t n, int64_t k,
               float* y, void* stream);

/*
 * Grouped (MoE) block-scaled W4A4 GEMM over a contiguous per-expert layout
 * with device-side metadata.
 *
 * Defined by: "miniTE报告" section Transformer Engine路径优化 (contiguous
 * layouts, device-side metadata, amax reuse and grouped GEMM for the
 * per-token NVFP4 path) and the Miles page, section 配方2 (NVFP4 on the MoE
 * expert layers).
 *
 *   A: a_q [a_rows, k/2], a_sb [a_rows, k/16], a_s [a_rows]
 *   row_index NULL: output row i reads A row i (then a_rows >= m_total).
 *             else [m_total] i32 device: output row i reads A row
 *             row_index[i] -- a token quantized once serves all its routed
 *             copies.  Indices outside [0, a_rows) read as zero rows.
 *   offsets   [groups+1] i32 device, non-decreasing: expert g owns output
 *             rows [offsets[g], offsets[g+1]).  Values are clamped to
 *             [0, m_total]; rows at or past offsets[groups] are not written.
 *   B: b_q [groups, n, k/2], b_sb [groups, n, k/16], b_s [groups] (per expert)
 *   y  [m_total, n] f32 out
 * Accuracy as nvfp4_gemm.  groups <= 1024.  Determinism as nvfp4_gemm.  The
 * kernel choice follows the whole layout: at most 16 routed rows per expert
 * on average (m_total <= 16 groups) with k % 256 == 0 takes the few-rows
 * kernel.
 * Errors: INVALID_VALUE (groups < 1, negative sizes, null pointers),
 * UNSUPPORTED_SHAPE (k % 16 != 0, groups > 1024), MISALIGNED, ARCH, LAUNCH.
 */
int nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s, int64_t a_rows,
                       const int32_t* row_index, int64_t m_total, const int32_t* offsets,
                       int64_t groups, const uint8_t* b_q, const uint8_t* b_sb, const float* b_s,
                       int64_t n, int64_t k, float* y, void* stream);

/*
 * Grouped (MoE) up-projection with SwiGLU in the epilogue: the fused gate|up
 * GEMM of nvfp4_grouped_gemm, but instead of the fp32 output Y [m_total, 2f]
 * it writes H = silu(gate) * up as bf16 and the row amax of H, the input of
 * the per-token requantize with amax reuse (nvfp4_quantize_rows with
 * amax_in = amax gives the same bits as quantizing H afresh).
 *
 * Defined by: "miniTE报告" section Transformer Engine路径优化 (fusion and amax
 * reuse around the low-precision GEMMs), the Miles page, section
 * 并行度与张量转换的一致性契约 (gate and up as one fused GEMM under one FP32
 * scale) and section 实验结果 item 10 (work fused into the GEMM epilogue).
 *
 *   A, row_index, offsets, groups: as nvfp4_grouped_gemm.
 *   B: b_q [groups, 2f, k/2], b_sb [groups, 2f, k/16], b_s [groups]: rows
 *      [0, f) of each expert are gate, rows [f, 2f) up.
 *   h    [m_total, f] bf16 out: h = bf16(fl32(g u / (1 + e^-g))) with the
 *        arithmetic of nvfp4_swiglu_quantize_rows, where g = Y[row, c] and
 *        u = Y[row, f + c] are the fused GEMM's fp32 outputs (accuracy as
 *        nvfp4_grouped_gemm; bit-identical to what nvfp4_grouped_gemm writes
 *        whenever that call takes its tiled kernel, i.e. more than 16 routed
 *        rows per expert on average).  Rows at or past offsets[groups] are
 *        not written.
 *   amax [m_total] f32 out: the largest |h| of each row (0 for rows past
 *        offsets[groups]).  Set to zero, then raised by atomic maxima of
 *        the bit patterns (the result does not depend on their order).
 * k must be a positive multiple of 256; 2f < 2^22.
 * Cost: it moves about 117 MB less HBM traffic than nvfp4_grouped_gemm plus
 * nvfp4_swiglu_quantize_rows on the MoE up-projection (and needs no fp32
 * output buffer), but on MI355X it takes longer: the SwiGLU arithmetic runs
 * in each tile's epilogue at one wave per SIMD, where the separate
 * HBM-bound SwiGLU kernel hides it behind memory traffic.
 * Errors: INVALID_VALUE, UNSUPPORTED_SHAPE (k, f or groups out of range),
 * MISALIGNED (codes and block scales 16 bytes, h 2, the rest 4), ARCH,
 * LAUNCH.
 */
int nvfp4_grouped_gemm_swiglu(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s,
                              int64_t a_rows, const int32_t* row_index, int64_t m_total,
                              const int32_t* offsets, int64_t groups, const uint8_t* b_q,
                              const uint8_t* b_sb, const float* b_s, int64_t f, int64_t k,
                              uint16_t* h, float* amax, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
