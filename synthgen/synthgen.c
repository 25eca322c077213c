/*
 * synthgen.c -- seeded synthetic inputs shared by the tests, the benchmark and
 * the oracle's self-checks.
 *
 * This file holds no part of the quantizer or GEMM arithmetic.  It only draws
 * random numbers and rounds them to bf16 storage:
 *
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): a counter-based stream, so element i of a
 *     stream is computable on its own and the output does not depend on the
 *     number of threads.
 *   - Box-Muller normals in fp64.
 *   - Student-t with nu = 3 as Z / sqrt(chi2_3 / 3), chi2_3 the sum of three
 *     squared normals, optionally scaled by 1/sqrt(3) to unit variance.
 *   - bf16 storage: fp64 -> fp32 (C cast, round to nearest even) -> bf16
 *     (round to nearest even on the fp32 bit pattern).  Inputs are finite.
 *
 * Streams: stream_base(seed, stream) picks an independent SplitMix64 start
 * state per (seed, tensor) pair; u64(seed, stream, i) is the i-th output.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see synthgen/__init__.py).
 */
#include <stdint.h>
#include <math.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ mix64(stream + 0x632BE59BD9B4E019ULL));
}

/* i-th output of SplitMix64 started at state `base` */
static inline uint64_t u64_at(uint64_t base, uint64_t i) {
    return mix64(base + (i + 1) * GOLDEN_GAMMA);
}

/* uniform in the open interval (0, 1) */
static inline double unif_at(uint64_t base, uint64_t i) {
    return ((double)(u64_at(base, i) >> 11) + 0.5) * 0x1.0p-53;
}

/* i-th standard normal of the stream: Box-Muller on uniform pair i/2 */
static inline double normal_at(uint64_t base, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = unif_at(base, 2 * p), u2 = unif_at(base, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f64_to_bf16(double v) {
    float f = (float)v;
    union { float f; uint32_t u; } c = { f };
    uint32_t u = c.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t i) {
    return u64_at(stream_base(seed, stream), i);
}

void synth_uniform_f64(uint64_t seed, uint64_t stream, int64_t n, double* out) {
    uint64_t b = stream_base(seed, stream);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = unif_at(b, (uint64_t)i);
}

void synth_normal_f64(uint64_t seed, uint64_t stream, int64_t n, double* out) {
    uint64_t b = stream_base(seed, stream);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = normal_at(b, (uint64_t)i);
}

/* N(mean, std^2), stored as bf16 bits */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double mean, double std,
                       uint16_t* out) {
    uint64_t b = stream_base(seed, stream);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f64_to_bf16(mean + std * normal_at(b, (uint64_t)i));
}

/* Student-t(3) times `scale` (scale = 1/sqrt(3) gives unit std), as bf16 bits */
void synth_student_t3_bf16(uint64_t seed, uint64_t stream, int64_t n, double scale,
                           uint16_t* out) {
    uint64_t b = stream_base(seed, stream);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t j = 4 * (uint64_t)i;
        double z = normal_at(b, j);
        double c = 0.0;
        for (int t = 1; t <= 3; ++t) { double g = normal_at(b, j + t); c += g * g; }
        out[i] = f64_to_bf16(scale * z / sqrt(c / 3.0));
    }
}

/* N(0, std^2) where each entry is multiplied by `mult` with probability `p`
 * (Bernoulli per entry from its own stream), stored as bf16 bits */
void synth_normal_outliers_bf16(uint64_t seed, uint64_t stream, int64_t n, double std,
                                double p, double mult, uint16_t* out) {
    uint64_t b = stream_base(seed, stream);
    uint64_t bo = stream_base(seed, stream + 0x100000000ULL);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = std * normal_at(b, (uint64_t)i);
        if (unif_at(bo, (uint64_t)i) < p) v *= mult;
        out[i] = f64_to_bf16(v);
    }
}

/* fp32 -> bf16 bits with round-to-nearest-even (finite inputs), for
 * hand-built inputs in tests */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f64_to_bf16((double)in[i]);
}
