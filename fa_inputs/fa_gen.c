/*
 * Seeded synthetic inputs: the definition in include/fa_gen.h, in plain C.
 * No attention arithmetic lives here; the GPU library and the CPU oracle both
 * read what these functions write.
 */
#include "fa_gen.h"

#include <math.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define MIX1 0xBF58476D1CE4E5B9ULL
#define MIX2 0x94D049BB133111EBULL
#define KEY_STREAM 0xD1B54A32D192ED03ULL
#define PI_D 3.14159265358979323846   /* rounds to the double nearest pi */

uint64_t fa_gen_key(uint64_t seed, uint64_t stream) { return (seed * GOLDEN) ^ ((stream + 1) * KEY_STREAM); }

uint64_t fa_gen_splitmix64(uint64_t key, uint64_t c) {
    uint64_t z = key + (c + 1) * GOLDEN;
    z = (z ^ (z >> 30)) * MIX1;
    z = (z ^ (z >> 27)) * MIX2;
    return z ^ (z >> 31);
}

static double uniform(uint64_t key, uint64_t c) {
    return ((double)(fa_gen_splitmix64(key, c) >> 11) + 0.5) * 0x1p-53;
}

static double normal(uint64_t key, uint64_t i, double sigma) {
    const double u1 = uniform(key, 2 * i), u2 = uniform(key, 2 * i + 1);
    return sigma * (sqrt(-2.0 * log(u1)) * cos(2.0 * PI_D * u2));
}

static uint16_t f32_to_bf16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    return (uint16_t)((x + 0x7FFFu + ((x >> 16) & 1u)) >> 16);
}

static uint16_t f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const uint32_t ax = x & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return sign | 0x7E00u;        /* NaN */
    if (ax >= 0x477FF000u) return sign | 0x7C00u;       /* >= 65520 rounds to infinity */
    if (ax >= 0x38800000u) {                            /* >= 2^-14: a normal binary16 */
        const uint32_t r = ax + 0xFFFu + ((ax >> 13) & 1u);   /* ties to even at bit 13 */
        return sign | (uint16_t)((r - (112u << 23)) >> 13);  /* exponent bias 127 -> 15 */
    }
    /* subnormal or zero: m * 2^-24 with m = |f| * 2^24 (exact) rounded to even */
    const float s = fabsf(f) * 16777216.0f;
    return sign | (uint16_t)nearbyintf(s);
}

void fa_gen_f32_to_f16(const float* src, uint16_t* dst, size_t n) {
    for (size_t i = 0; i < n; ++i) dst[i] = f32_to_f16(src[i]);
}

void fa_gen_f32_to_bf16(const float* src, uint16_t* dst, size_t n) {
    for (size_t i = 0; i < n; ++i) dst[i] = f32_to_bf16(src[i]);
}

int fa_gen_normal(double* dst, size_t start, size_t n, uint64_t seed, uint64_t stream, double sigma) {
    if (n > 0 && !dst) return -1;
    const uint64_t key = fa_gen_key(seed, stream);
    const long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long j = 0; j < nn; ++j) dst[j] = normal(key, (uint64_t)start + (uint64_t)j, sigma);
    return 0;
}

int fa_gen_fill_range(void* dst, int dtype, size_t start, size_t n, uint64_t seed, uint64_t stream,
                      double sigma) {
    if (dtype < 0 || dtype > 2) return -2;
    if (n > 0 && !dst) return -1;
    const uint64_t key = fa_gen_key(seed, stream);
    const long long nn = (long long)n;
    if (dtype == 0) {
        float* out = (float*)dst;
#pragma omp parallel for schedule(static)
        for (long long j = 0; j < nn; ++j) out[j] = (float)normal(key, (uint64_t)start + (uint64_t)j, sigma);
    } else {
        uint16_t* out = (uint16_t*)dst;
        const int half = dtype == 1;
#pragma omp parallel for schedule(static)
        for (long long j = 0; j < nn; ++j) {
            const float v = (float)normal(key, (uint64_t)start + (uint64_t)j, sigma);
            out[j] = half ? f32_to_f16(v) : f32_to_bf16(v);
        }
    }
    return 0;
}

int fa_gen_fill(void* dst, int dtype, size_t n, uint64_t seed, uint64_t stream, double sigma) {
    return fa_gen_fill_range(dst, dtype, 0, n, seed, stream, sigma);
}
