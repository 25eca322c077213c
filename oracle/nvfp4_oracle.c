/*
 * nvfp4_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the per-token NVFP4
 * path computes.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; the product library never does, and the two share no
 * source, header, table or helper.
 *
 * Sources (titles of the pages the method is described on):
 *  [P1] "miniTE报告：原生NVFP4训RL后期为何失稳，8×B300上提速1.37倍", section
 *       "NVFP4格式、两级缩放与转换误差": values are E2M1 (1 sign bit, E exponent
 *       bits, M mantissa bits), each 16 elements share an E4M3 block scale s_b,
 *       and an FP32 outer scale sits above it (per tensor, per expert or per row).
 *  [P4] "Towards Blackwell-Native 8-bit and 4-bit RL: End-to-End MXFP8 and
 *       NVFP4 RL in Miles": section 速读 / 怎么做的 gives X ~ s_token * s_block *
 *       X_FP4 with 16 E2M1 values per E4M3 block scale and s_token computed
 *       online per token; section 背景知识与设计原则 / NVFP4格式背景 says the E4M3
 *       scale is rounded to the nearest representable value and the FP32 scale
 *       maps the tensor or token into NVFP4's representable range; section
 *       方法细节 / 位级精确的量化器契约 asks for byte-exact quantizers; section
 *       服务与RL在量化上的实际区别 rules out fast-math; the recipe in 补充细节
 *       disables stochastic rounding.
 *  [P5] "TRIAGE: Direction-Aware Mismatch Stabilization of Native NVFP4
 *       Reinforcement Learning", section 前置知识 / NVFP4 量化格式与 W4A4 执行:
 *       decode x_hat_j = S * s_b * Q_E2M1(x_j / (S * s_b)).
 *
 * Readings taken where the pages leave a step open (each is listed with its
 * reason in the design notes of the repository):
 *  - outer scale S = fl32(amax / 2688), 2688 = 6 (E2M1 max) * 448 (E4M3 max);
 *  - block scale s_b = RNE_SAT_E4M3(fl32(a_b / fl32(6 * S))), s_b = 0 when S = 0;
 *  - element code = RNE_SAT_E2M1(|fl32(x * fl32(1 / fl32(S * s_b)))|) with the
 *    sign bit copied from x, and magnitude 0 when S * s_b == 0 or x == +-0;
 *  - RNE_SAT(v): nearest finite code value, ties to the even code, +inf and
 *    values above the maximum give the maximum;
 *  - E4M3 is the OCP "FN" variant (bias 7, max 448, 0x7F/0xFF are NaN);
 *  - pack: element 2i in the low nibble of byte i, element 2i+1 in the high one;
 *  - block scales row-major [rows, K/16], outer scales fp32.
 * All fp32 steps are single IEEE operations (built with -ffp-contract=off, no
 * fast-math, denormals kept).
 *
 * GEMM: Y[m,n] = S_A[m] * S_B * sum_k u_A[m,k] * u_B[n,k] with u = s_b * e2m1(q).
 * Every u times 2^10 is an integer of magnitude <= 2688 * 1024, so the sum is
 * formed exactly in int64 and scaled in fp64 at the end.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <omp.h>

/* number of OpenMP threads the parallel loops below use, and a way to set it
 * (the CPU baseline times the quantizer on one thread as well as on all) */
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ---------------------------------------------------------------- codecs -- */

/* E2M1 code (4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit) */
double oracle_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -mag : mag;
}

/* E4M3 "FN" code (sign, 4 exponent bits with bias 7, 3 mantissa bits); NaN for
 * the all-ones exponent and mantissa */
double oracle_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest non-negative finite code to v >= 0 (v may be +inf); on a tie the
 * code with an even bit pattern wins.  Brute force over every code. */
static int rne_sat_search(double v, int ncodes, double (*value)(int)) {
    int best = -1;
    double bestd = 0.0, maxv = -1.0;
    int maxc = 0;
    for (int c = 0; c < ncodes; ++c) {
        double t = value(c);
        if (isnan(t)) continue;
        if (t > maxv) { maxv = t; maxc = c; }
    }
    if (isinf(v) || v >= maxv) return maxc;
    for (int c = 0; c < ncodes; ++c) {
        double t = value(c);
        if (isnan(t)) continue;
        double d = fabs(v - t);
        if (best < 0 || d < bestd || (d == bestd && (c & 1) == 0)) { best = c; bestd = d; }
    }
    return best;
}

/* non-negative codes only: 0..7 for E2M1, 0..127 for E4M3 */
int oracle_rne_sat_e2m1(float v) { return rne_sat_search((double)v, 8, oracle_e2m1_value); }
int oracle_rne_sat_e4m3(float v) { return rne_sat_search((double)v, 128, oracle_e4m3_value); }

void oracle_rne_sat_e2m1_array(const float* v, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_rne_sat_e2m1(v[i]);
}
void oracle_rne_sat_e4m3_array(const float* v, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_rne_sat_e4m3(v[i]);
}

/* bf16 bit pattern -> fp32 (exact: bf16 is the top half of an fp32) */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------- quantizer -- */

/* Encode one row of k elements given its fp32 outer scale S. */
static void encode_row(const uint16_t* x, int64_t k, float S, uint8_t* q, uint8_t* sb) {
    int64_t nblk = k / 16;
    for (int64_t b = 0; b < nblk; ++b) {
        float xs[16];
        float ab = 0.0f;
        for (int j = 0; j < 16; ++j) {
            xs[j] = bf16_to_f32(x[16 * b + j]);
            float a = fabsf(xs[j]);
            if (a > ab) ab = a;
        }
        /* block scale */
        int sc;
        if (S == 0.0f) {
            sc = 0;
        } else {
            float t = 6.0f * S;
            float v = ab / t;
            sc = oracle_rne_sat_e4m3(v);
        }
        sb[b] = (uint8_t)sc;
        /* element codes */
        float sbv = (float)oracle_e4m3_value(sc);
        float d = S * sbv;
        float inv = (d != 0.0f) ? 1.0f / d : 0.0f;
        uint8_t codes[16];
        for (int j = 0; j < 16; ++j) {
            int mag;
            if (d == 0.0f || xs[j] == 0.0f) {
                mag = 0;
            } else {
                float r = xs[j] * inv;
                mag = oracle_rne_sat_e2m1(fabsf(r));
            }
            codes[j] = (uint8_t)((signbit(xs[j]) ? 8 : 0) | mag);
        }
        for (int j = 0; j < 8; ++j)
            q[8 * b + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
    }
}

static float row_amax(const uint16_t* x, int64_t k) {
    float a = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
        float v = fabsf(bf16_to_f32(x[j]));
        if (v > a) a = v;
    }
    return a;
}

/* Per-token quantization: one FP32 outer scale per row from the row amax
 * (or from amax_in[r] when given).  Returns 0, or -1 on a bad shape or a
 * non-finite input. */
int oracle_quantize_rows(const uint16_t* x, int64_t rows, int64_t k, const float* amax_in,
                         uint8_t* q, uint8_t* sb, float* s) {
    if (rows < 0 || k < 0 || k % 16 != 0) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * k;
        for (int64_t j = 0; j < k; ++j)
            if (((xr[j] >> 7) & 0xFF) == 0xFF) bad = 1;
        float amax = amax_in ? amax_in[r] : row_amax(xr, k);
        float S = amax / 2688.0f;
        s[r] = S;
        encode_row(xr, k, S, q + r * (k / 2), sb + r * (k / 16));
    }
    return bad ? -1 : 0;
}

/* Weight quantization: groups x rows_per_group rows; one FP32 outer scale per
 * group (per tensor when groups == 1, per expert otherwise) from the group
 * amax (or amax_in[g]).  amax_out may be NULL. */
int oracle_quantize_weight(const uint16_t* w, int64_t groups, int64_t rows_per_group, int64_t k,
                           const float* amax_in, float* amax_out, uint8_t* q, uint8_t* sb,
                           float* s) {
    if (groups < 0 || rows_per_group < 0 || k < 0 || k % 16 != 0) return -1;
    int bad = 0;
    for (int64_t g = 0; g < groups; ++g) {
        const uint16_t* wg = w + g * rows_per_group * k;
        float amax = 0.0f;
        if (amax_in) {
            amax = amax_in[g];
        } else {
            #pragma omp parallel for schedule(static) reduction(max : amax)
            for (int64_t r = 0; r < rows_per_group; ++r) {
                float a = row_amax(wg + r * k, k);
                if (a > amax) amax = a;
            }
        }
        if (amax_out) amax_out[g] = amax;
        float S = amax / 2688.0f;
        s[g] = S;
        #pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
        for (int64_t r = 0; r < rows_per_group; ++r) {
            const uint16_t* xr = wg + r * k;
            for (int64_t j = 0; j < k; ++j)
                if (((xr[j] >> 7) & 0xFF) == 0xFF) bad = 1;
            int64_t row = g * rows_per_group + r;
            encode_row(xr, k, S, q + row * (k / 2), sb + row * (k / 16));
        }
    }
    return bad ? -1 : 0;
}

/* Decode: x_hat = S * s_b * e2m1(q), in fp64 (exact).  s_index[r] selects the
 * outer scale of row r (row r for per-token scales, the group for weights). */
void oracle_dequantize(const uint8_t* q, const uint8_t* sb, const float* s,
                       const int64_t* s_index, int64_t rows, int64_t k, double* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double S = (double)s[s_index ? s_index[r] : r];
        for (int64_t j = 0; j < k; ++j) {
            uint8_t byte = q[r * (k / 2) + j / 2];
            int code = (j & 1) ? (byte >> 4) : (byte & 15);
            double sbv = oracle_e4m3_value(sb[r * (k / 16) + j / 16]);
            out[r * k + j] = S * sbv * oracle_e2m1_value(code);
        }
    }
}

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 bit pattern nearest to the fp32 value v (IEEE round to nearest, ties to
 * the even pattern).  Truncating v's low 16 bits gives the neighbour on the
 * zero side; the pattern one above it is the neighbour away from zero (past
 * the largest finite bf16 that neighbour is infinity, which rounding treats as
 * the value 2^128, so halfway and beyond overflow as IEEE requires).  v must
 * not be NaN. */
static uint16_t f32_to_bf16_nearest(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0) return lo;
    uint16_t hi = (uint16_t)(lo + 1);
    double lv = bf16_to_f32(lo);
    double hv = ((hi & 0x7FFF) == 0x7F80) ? copysign(ldexp(1.0, 128), v) : bf16_to_f32(hi);
    double dl = fabs((double)v - lv), dh = fabs(hv - (double)v);
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

/* bf16 bit pattern nearest to a finite double x (ties to the even pattern;
 * values at or past the halfway point above the largest bf16 give infinity).
 * The bf16 grid near x has spacing 2^(e - 7) where 2^e <= |x| < 2^(e+1),
 * e >= -126 (below that the subnormal spacing 2^-133); the two grid points
 * around |x| are found by exact power-of-two scaling and floor. */
static uint16_t f64_to_bf16_nearest(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);         /* a = f * 2^e, 0.5 <= f < 1 */
    e -= 1;               /* 2^e <= a < 2^(e+1) */
    if (e < -126) e = -126;
    double ulp = ldexp(1.0, e - 7);
    double m = floor(a / ulp);          /* grid index of the lower neighbour */
    double lo = m * ulp, hi = (m + 1.0) * ulp;
    double dl = a - lo, dh = hi - a;    /* exact: a has far fewer bits than a double */
    double r = (dl < dh) ? m : (dh < dl) ? m + 1.0 : (fmod(m, 2.0) == 0.0 ? m : m + 1.0);
    double v = r * ulp;
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    /* bit pattern of the finite bf16 value v */
    float fv = (float)v;                /* exact: v is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &fv, 4);
    return (uint16_t)(sign | (u >> 16));
}

void oracle_f64_to_bf16_array(const double* v, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f64_to_bf16_nearest(v[i]);
}

void oracle_f32_to_bf16_array(const float* v, int64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_nearest(v[i]);
}

/* -------------------------------------------------------------- SwiGLU -- */

/* SwiGLU over a fused gate|up row block (the pages' MoE layers fuse the gate
 * and up projections into one GEMM sharing one FP32 weight scale: Miles page,
 * section 并行度与张量转换的一致性契约; SwiGLU itself is silu(gate) * up, with
 * silu(g) = g * sigmoid(g) = g / (1 + e^-g), Shazeer, "GLU Variants Improve
 * Transformer", 2020).
 *
 * gate_up is fp32 [rows, 2f]: columns [0, f) hold the gate projection and
 * [f, 2f) the up projection of the same token.  Output h is bf16 [rows, f]:
 * h = bf16(fl32(silu(g) * u)), the real value evaluated in fp64 as
 * (g * u) / (1 + exp(-g)) (g * u is exact in fp64), rounded once to fp32 and
 * then to bf16, both to nearest even.  Returns -1 on a bad shape, a
 * non-finite input or a result that is not finite in fp32, else 0. */
int oracle_swiglu_rows(const float* gate_up, int64_t rows, int64_t f, uint16_t* h) {
    if (rows < 0 || f < 0) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        const float* gr = gate_up + r * 2 * f;
        for (int64_t j = 0; j < f; ++j) {
            double g = gr[j], u = gr[f + j];
            if (!isfinite(g) || !isfinite(u)) { bad = 1; h[r * f + j] = 0; continue; }
            double hv = (g * u) / (1.0 + exp(-g));
            float h32 = (float)hv;
            if (!isfinite(h32)) { bad = 1; h[r * f + j] = 0; continue; }
            h[r * f + j] = f32_to_bf16_nearest(h32);
        }
    }
    return bad ? -1 : 0;
}

/* -------------------------------------------------------------- routing -- */

/* Top-k MoE routing into the contiguous per-expert layout (miniTE page,
 * section Transformer Engine路径优化: contiguous layouts and device-side
 * metadata for the grouped GEMMs; the layers route each token to its top-k
 * experts by router logit, softmax being monotone).
 *
 * logits fp32 [T, E], finite.  For token t, experts[t, j] (j < topk) is the
 * expert with the j-th largest logit; equal logits rank the lower expert id
 * first (+0 and -0 are equal).  The T * topk (token, expert) pairs are then
 * ordered by expert, and by token within an expert: offsets[e] is the number
 * of pairs with a smaller expert id (offsets[E] = T * topk), the pair at
 * position p has token row_index[p], and slot_of[t, j] is the position of the
 * pair (t, experts[t, j]).  Returns -1 on a bad shape or a non-finite logit. */
int oracle_route(const float* logits, int64_t T, int64_t E, int64_t topk, int32_t* experts,
                 int32_t* offsets, int32_t* row_index, int32_t* slot_of) {
    if (T < 0 || E < 1 || topk < 1 || topk > E) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t t = 0; t < T; ++t) {
        const float* lt = logits + t * E;
        for (int64_t e = 0; e < E; ++e)
            if (!isfinite(lt[e])) bad = 1;
        for (int64_t j = 0; j < topk; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int64_t i = 0; i < j; ++i)
                    if (experts[t * topk + i] == e) taken = 1;
                if (taken) continue;
                /* strictly greater wins, so among equal logits the lowest id stays */
                if (best < 0 || lt[e] > lt[best]) best = e;
            }
            experts[t * topk + j] = (int32_t)best;
        }
    }
    if (bad) return -1;
    int64_t p = 0;
    for (int64_t e = 0; e < E; ++e) {
        offsets[e] = (int32_t)p;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < topk; ++j)
                if (experts[t * topk + j] == e) {
                    row_index[p] = (int32_t)t;
                    slot_of[t * topk + j] = (int32_t)p;
                    ++p;
                }
    }
    offsets[E] = (int32_t)p;
    return 0;
}

/* Dequantize to bf16, for backward GEMMs that consume the dequantized
 * forward operands (Miles page, section 反量化反向模式: the backward runs in
 * BF16 on the BF16 dequantization of the exact low-precision operands):
 * x_bf16 = bf16(S * s_b * e2m1(q)), the product formed exactly (at most 30
 * significant bits) and rounded once to nearest even.  Row r uses the outer
 * scale s[r / rows_per_scale] (1 for per-token scales, the group's row count
 * for per-tensor / per-expert weights). */
void oracle_dequantize_bf16(const uint8_t* q, const uint8_t* sb, const float* s,
                            int64_t rows, int64_t k, int64_t rows_per_scale, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double S = (double)s[r / rows_per_scale];
        for (int64_t j = 0; j < k; ++j) {
            uint8_t byte = q[r * (k / 2) + j / 2];
            int code = (j & 1) ? (byte >> 4) : (byte & 15);
            double sbv = oracle_e4m3_value(sb[r * (k / 16) + j / 16]);
            out[r * k + j] = f64_to_bf16_nearest(S * sbv * oracle_e2m1_value(code));
        }
    }
}

/* ---------------------------------------------------------------- MXFP8 -- */

/* MXFP8 (Miles page, section MXFP8格式背景): each run of 32 consecutive
 * values along the contraction axis is stored as E4M3 codes under one E8M0
 * scale, a power of two 2^e (code e + 127, codes 0..254).  The scale is
 * rounded up: 2^e is the smallest power of two with a_b / 2^e <= 448 (the
 * E4M3 maximum), so the block maximum is never clipped; an all-zero block
 * (and any block needing e < -127) takes code 0.  Elements are
 * RNE_SAT_E4M3(|x| / 2^e) with the sign bit of x (bit 7).
 * x is bf16 [rows, k], k % 32 == 0.  q [rows, k] E4M3 codes, sc [rows, k/32].
 * Returns -1 on a bad shape or a non-finite input, else 0. */
static int mx_scale_exponent(double amax) {
    if (amax == 0.0) return -127;
    int e = -127;
    while (ldexp(448.0, e) < amax) ++e;   /* smallest e with amax <= 448 * 2^e */
    return e;
}

int oracle_mxfp8_quantize_rows(const uint16_t* x, int64_t rows, int64_t k, uint8_t* q,
                               uint8_t* sc) {
    if (rows < 0 || k < 0 || k % 32 != 0) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < k / 32; ++b) {
            const uint16_t* xb = x + r * k + 32 * b;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                double v = fabs((double)bf16_to_f32(xb[j]));
                if (!isfinite(v)) bad = 1;
                if (v > amax) amax = v;
            }
            int e = mx_scale_exponent(amax);
            sc[r * (k / 32) + b] = (uint8_t)(e + 127);
            for (int j = 0; j < 32; ++j) {
                float xv = bf16_to_f32(xb[j]);
                /* |x| / 2^e is exact in double; the E4M3 search rounds it */
                double v = ldexp(fabs((double)xv), -e);
                int mag = rne_sat_search(v, 128, oracle_e4m3_value);
                q[r * k + 32 * b + j] = (uint8_t)((signbit(xv) ? 0x80 : 0) | mag);
            }
        }
    }
    return bad ? -1 : 0;
}

/* MXFP8 GEMM reference: Y[m,n] = sum over blocks of 2^(e_A + e_B) * sum of
 * the 32 products of E4M3 values.  Within a block the products are integers
 * times 2^-18 and their sum is formed exactly in int64; the blocks are summed
 * in fp64 (error at most (k/32) * 2^-53 * sum |a b|).  bound = sum |a_k b_k|
 * in fp64.  A [m, k] codes + [m, k/32] scales, B [n, k] + [n, k/32]. */
static int64_t e4m3_int(uint8_t c) {   /* E4M3 value * 2^9, exact integer */
    double v = oracle_e4m3_value(c & 0x7F) * 512.0;
    int64_t iv = (int64_t)v;
    return (c & 0x80) ? -iv : iv;
}

void oracle_mxfp8_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t m, const uint8_t* b_q,
                       const uint8_t* b_sc, int64_t n, int64_t k, double* y, double* bound) {
    int64_t nb = k / 32;
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, bnd = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int64_t s = 0, sa = 0;
                for (int t = 0; t < 32; ++t) {
                    int64_t p = e4m3_int(a_q[i * k + 32 * b + t]) * e4m3_int(b_q[j * k + 32 * b + t]);
                    s += p;
                    sa += p < 0 ? -p : p;
                }
                int ex = (int)a_sc[i * nb + b] + (int)b_sc[j * nb + b] - 254 - 18;
                acc += ldexp((double)s, ex);
                bnd += ldexp((double)sa, ex);
            }
            y[i * n + j] = acc;
            bound[i * n + j] = bnd;
        }
    }
}

/* ------------------------------------------------------------------ GEMM -- */

/* s_b * e2m1(code) * 2^10 as an exact integer, tabulated once per call for
 * every (scale code, element code) pair; scale codes 0x7F/0xFF (NaN) never
 * occur in a quantized operand and map to 0 here */
static int64_t unit_table[256][16];

static void fill_unit_table(void) {
    for (int sc = 0; sc < 256; ++sc)
        for (int c = 0; c < 16; ++c) {
            double v = oracle_e4m3_value(sc);
            unit_table[sc][c] = isnan(v) ? 0 : (int64_t)(v * oracle_e2m1_value(c) * 1024.0);
        }
}

static int64_t unit_int(uint8_t sbcode, int code) { return unit_table[sbcode][code]; }

/* exact dot of row a (of A) and row b (of B) in units of 2^-20; also the
 * exact sum of absolute products */
static void dot_exact(const uint8_t* aq, const uint8_t* asb, const uint8_t* bq,
                      const uint8_t* bsb, int64_t k, int64_t* dot, int64_t* absdot) {
    int64_t acc = 0, aacc = 0;
    for (int64_t j = 0; j < k; ++j) {
        int ca = (j & 1) ? (aq[j / 2] >> 4) : (aq[j / 2] & 15);
        int cb = (j & 1) ? (bq[j / 2] >> 4) : (bq[j / 2] & 15);
        int64_t ua = unit_int(asb[j / 16], ca);
        int64_t ub = unit_int(bsb[j / 16], cb);
        int64_t p = ua * ub;
        acc += p;
        aacc += (p < 0) ? -p : p;
    }
    *dot = acc;
    *absdot = aacc;
}

/* Entry list form: for each i, Y_ref[i] = S_A[a_row[i]] * S_B[b_scale[i]] *
 * dot(A row a_row[i], B row b_row[i]); bound[i] = the same scales times the
 * sum of |products|.  Covers dense (b_scale = 0) and grouped GEMM. */
void oracle_gemm_entries(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s,
                         const uint8_t* b_q, const uint8_t* b_sb, const float* b_s, int64_t k,
                         const int64_t* a_row, const int64_t* b_row, const int64_t* b_scale,
                         int64_t count, double* y_ref, double* bound) {
    fill_unit_table();
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t dot, absdot;
        dot_exact(a_q + a_row[i] * (k / 2), a_sb + a_row[i] * (k / 16),
                  b_q + b_row[i] * (k / 2), b_sb + b_row[i] * (k / 16), k, &dot, &absdot);
        double sc = (double)a_s[a_row[i]] * (double)b_s[b_scale[i]] * 0x1.0p-20;
        y_ref[i] = sc * (double)dot;
        bound[i] = sc * (double)absdot;
    }
}

/* Dense: Y[m,n] = deq(A)[m,:] . deq(B)[n,:], A [m,k], B [n,k], per-tensor S_B */
void oracle_gemm(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s, int64_t m,
                 const uint8_t* b_q, const uint8_t* b_sb, const float* b_s, int64_t n, int64_t k,
                 double* y_ref, double* bound) {
    fill_unit_table();
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int64_t dot, absdot;
            dot_exact(a_q + i * (k / 2), a_sb + i * (k / 16), b_q + j * (k / 2),
                      b_sb + j * (k / 16), k, &dot, &absdot);
            double sc = (double)a_s[i] * (double)b_s[0] * 0x1.0p-20;
            y_ref[i * n + j] = sc * (double)dot;
            bound[i * n + j] = sc * (double)absdot;
        }
    }
}

/* Grouped: output rows [offsets[g], offsets[g+1]) use expert g's weight
 * B[g] ([n,k]) and scale b_s[g]; output row i reads A row row_index[i]
 * (or row i when row_index is NULL).  Rows at or past offsets[groups] are
 * not part of the product and are left untouched. */
void oracle_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sb, const float* a_s,
                         const int32_t* row_index, const int32_t* offsets, int64_t groups,
                         const uint8_t* b_q, const uint8_t* b_sb, const float* b_s, int64_t n,
                         int64_t k, double* y_ref, double* bound) {
    fill_unit_table();
    for (int64_t g = 0; g < groups; ++g) {
        int64_t lo = offsets[g], hi = offsets[g + 1];
        #pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = lo; i < hi; ++i) {
            int64_t ar = row_index ? row_index[i] : i;
            for (int64_t j = 0; j < n; ++j) {
                int64_t br = g * n + j, dot, absdot;
                dot_exact(a_q + ar * (k / 2), a_sb + ar * (k / 16), b_q + br * (k / 2),
                          b_sb + br * (k / 16), k, &dot, &absdot);
                double sc = (double)a_s[ar] * (double)b_s[g] * 0x1.0p-20;
                y_ref[i * n + j] = sc * (double)dot;
                bound[i * n + j] = sc * (double)absdot;
            }
        }
    }
}
