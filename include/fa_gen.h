/*
 * Seeded synthetic inputs for the attention library and its CPU oracle.
 *
 * The pages measure on no dataset (their workload names, "GPT-J 2K/4K/8K"
 * in "FlashAttention 深度解析", second article section 2.4, and "GPT-2, seq
 * 1K" in "FlashAttention: как реально считается attention на GPU", name
 * sequence lengths only), so every input here is an i.i.d. normal tensor of
 * the workload's shape.  This library holds no attention arithmetic: it turns
 * (seed, stream, element index) into numbers and rounds them to the storage
 * type that the GPU library and the oracle both read.  It is plain host C
 * (fa_inputs/fa_gen.c), built with gcc into fa_inputs/libfa_gen.so.
 *
 * Definition (counter-based: element i never depends on how many elements
 * were drawn before it, or on how a fill is split into ranges or threads):
 *   key      = seed * 0x9E3779B97F4A7C15 ^ (stream + 1) * 0xD1B54A32D192ED03
 *   raw(c)   = SplitMix64 finaliser (Steele, Lea and Flood, OOPSLA 2014) of
 *              key + (c + 1) * 0x9E3779B97F4A7C15                (mod 2^64)
 *   u(c)     = ((raw(c) >> 11) + 0.5) * 2^-53                    in (0, 1)
 *   z_i      = sqrt(-2 log u(2i)) * cos(2 pi u(2i+1))   Box-Muller, cosine
 *              branch, in double with the C library's log, cos and sqrt
 *   x_i      = sigma * z_i (double), rounded to float32 (round to nearest,
 *              ties to even), then for the 16-bit types rounded again to
 *              IEEE binary16 or bfloat16 (round to nearest, ties to even).
 *
 * Storage type codes are those of fa.h: 0 = float32, 1 = binary16,
 * 2 = bfloat16 (stored as its 16 raw bits).  Buffers are host memory owned by
 * the caller; element i of a fill is written at dst[i] (element size 4 or 2
 * bytes).  Every function is reentrant; the fills use OpenMP threads.
 *
 * Return codes: 0 on success, -1 for a null buffer with n > 0, -2 for an
 * unknown dtype.  Nothing is written on an error.
 */
#ifndef FA_GEN_H
#define FA_GEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The generator key of (seed, stream). */
uint64_t fa_gen_key(uint64_t seed, uint64_t stream);

/* raw(c) of the key: the SplitMix64 output with counter c. */
uint64_t fa_gen_splitmix64(uint64_t key, uint64_t c);

/* Elements 0 .. n-1 of (seed, stream), sigma * N(0,1), in storage type dtype. */
int fa_gen_fill(void* dst, int dtype, size_t n, uint64_t seed, uint64_t stream, double sigma);

/* Elements start .. start+n-1 of the same sequence (dst[j] = element start+j). */
int fa_gen_fill_range(void* dst, int dtype, size_t start, size_t n, uint64_t seed, uint64_t stream,
                      double sigma);

/* sigma * z_i in double (before any rounding) for i = start .. start+n-1. */
int fa_gen_normal(double* dst, size_t start, size_t n, uint64_t seed, uint64_t stream, double sigma);

/* The storage roundings on their own: float32 -> binary16 / bfloat16 bits
 * (round to nearest, ties to even; binary16 overflows to infinity). */
void fa_gen_f32_to_f16(const float* src, uint16_t* dst, size_t n);
void fa_gen_f32_to_bf16(const float* src, uint16_t* dst, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* FA_GEN_H */
