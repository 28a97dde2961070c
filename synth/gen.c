/*
 * Seeded synthetic inputs for the CSA2 workloads.
 *
 * This file holds input generation only: random numbers and the storage
 * conversions that turn them into the dtypes the workloads name (bf16 and
 * fp8 e4m3 for index vectors, bf16 for queries and window rows).  It holds
 * none of the method's arithmetic.  Both the CPU oracle and the GPU path are
 * fed from these bytes.
 *
 * Generator: counter-based SplitMix64.  Word n of stream `seed` is
 * mix(state0 + (n+1)*GAMMA) with state0 = mix(seed), where mix is the
 * SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as published in
 * Vigna's reference splitmix64.c).  Being counter-based, any element can be
 * produced independently, so large caches are generated in parallel and a
 * test can regenerate just the rows it samples.
 *
 * Normals: Box-Muller (Box & Muller 1958) on the word pair (2p, 2p+1):
 * u1 in (0,1], u2 in [0,1), r = sqrt(-2 ln u1); element 2p = r cos(2 pi u2),
 * element 2p+1 = r sin(2 pi u2), evaluated in fp64 and rounded to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_word(uint64_t seed, uint64_t n) {
    return sm64_mix(sm64_mix(seed) + (n + 1) * SM64_GAMMA);
}

static inline double normal_at(uint64_t state0, uint64_t g) {
    uint64_t p = g >> 1;
    uint64_t r1 = sm64_mix(state0 + (2 * p + 1) * SM64_GAMMA);
    uint64_t r2 = sm64_mix(state0 + (2 * p + 2) * SM64_GAMMA);
    double u1 = (double)((r1 >> 11) + 1) * 0x1p-53; /* (0, 1] */
    double u2 = (double)(r2 >> 11) * 0x1p-53;       /* [0, 1) */
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    return (g & 1) ? rad * sin(th) : rad * cos(th);
}

/* out[i] = element (offset + i) of the N(0,1) stream `seed`, as fp32. */
void synth_normal_f32(uint64_t seed, uint64_t offset, int64_t n, float* out) {
    const uint64_t s0 = sm64_mix(seed);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)normal_at(s0, offset + (uint64_t)i);
}

/* Rows of a [rows][row_len] block whose global row ids are given: element
   (row_ids[r]*row_len + c) of the stream.  Lets a test rebuild sampled rows. */
void synth_normal_rows_f32(uint64_t seed, const int64_t* row_ids, int64_t rows, int64_t row_len,
                           float* out) {
    const uint64_t s0 = sm64_mix(seed);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < row_len; ++c)
            out[r * row_len + c] = (float)normal_at(s0, (uint64_t)(row_ids[r] * row_len + c));
}

/* fp32 -> bf16 bits, IEEE round-to-nearest-even; NaN stays a quiet NaN. */
static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

/* fp32 -> OCP fp8 e4m3fn bits (bias 7, largest finite 448, no infinity),
   round-to-nearest-even, magnitudes >= 448 saturate to 448. */
static inline uint8_t f32_to_e4m3(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return sign | 0x7f;
    float a = fabsf(f);
    if (a >= 448.0f) return sign | 0x7e;
    if (a == 0.0f) return sign;
    int e;
    frexpf(a, &e);
    e -= 1; /* a = m * 2^e, m in [1,2) */
    if (e < -6) e = -6; /* subnormal range shares the quantum 2^-9 */
    float n = ldexpf(a, 3 - e); /* a / quantum, exact */
    float rn = nearbyintf(n);   /* ties to even under the default rounding mode */
    int code = ((e + 7) << 3) + (int)rn - 8;
    return sign | (uint8_t)code;
}

void synth_to_bf16(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(x[i]);
}

void synth_to_e4m3(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_e4m3(x[i]);
}

/* Fused: N(0,1) stream straight to bf16 / e4m3 without an fp32 buffer. */
void synth_normal_bf16(uint64_t seed, uint64_t offset, int64_t n, uint16_t* out) {
    const uint64_t s0 = sm64_mix(seed);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16((float)normal_at(s0, offset + (uint64_t)i));
}

void synth_normal_e4m3(uint64_t seed, uint64_t offset, int64_t n, uint8_t* out) {
    const uint64_t s0 = sm64_mix(seed);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_e4m3((float)normal_at(s0, offset + (uint64_t)i));
}
