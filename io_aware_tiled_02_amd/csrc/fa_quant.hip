// FP8 (E4M3) block quantisation of Q or K for the FP8 forward pass, gfx950.
//
// "FlashAttention 深度解析", third article (FlashAttention-3), section 2.3:
// Q and K are cut into blocks and each block is scaled into the FP8 range on
// its own, s = max|block| / FP8_MAX, codes = Quantize(block / s); the scores
// are dequantised after the product with s_q * s_k.  E4M3 is the OCP 8-bit
// format (bias 7, no infinities, largest finite value 448), which is what
// gfx950's v_cvt_pk_fp8_f32 produces, rounding to nearest even.
//
// A block is `block` consecutive rows of one (batch, head), all d columns:
// one contiguous span of the (B, H, L, d) tensor.  One workgroup per block
// loads it into registers, reduces the maximum and converts what it holds,
// so the kernel moves 2 + 1 bytes of HBM per element.  Blocks beyond 16K
// elements take a second kernel that reads the block twice instead of holding
// it; keeping the two apart leaves the common kernel free of a branch on the
// block size, which lets all of its loads issue before the first wait.  The
// arithmetic is float32:
// s = amax / 448 and x / s are IEEE-rounded divisions, and the quotient is
// clamped to +-448 before conversion (the conversion does not saturate; the
// clamp only absorbs the rounding of s).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace {

using namespace fa_dev;

constexpr float kE4M3Max = 448.f;

// Pieces (16 bytes, 8 elements) per thread kept in registers between the
// two passes: blocks up to 256 * kKeep pieces (128 rows at d = 128) read HBM
// once; larger blocks read it twice.
constexpr int kKeep = 8;

// x is read once (its last read, in the two-pass kernel) and x8 written once:
// those accesses carry the nontemporal hint, so the stream does not displace
// cached lines (21 -> 19 us per 64 MiB bf16 tensor, results bitwise equal)
__device__ inline u32x4 ld16_streamed(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <class T>
__device__ inline void quant_store(const u32x4 raw, float s, unsigned char* dst) {
    float v[8];
    load_elems<T, 8>(reinterpret_cast<const char*>(&raw), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf(v[e] / s, -kE4M3Max), kE4M3Max);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
    __builtin_nontemporal_store(u32x2{(uint32_t)w0, (uint32_t)w1}, reinterpret_cast<u32x2*>(dst));
}

template <class T>
__device__ inline float piece_amax(const u32x4 raw) {
    float v[8];
    load_elems<T, 8>(reinterpret_cast<const char*>(&raw), v);
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    return m;
}

// Blocks of at most 256 * kKeep pieces: held in registers, HBM read once.
template <class T>
__global__ __launch_bounds__(256) void fa_quant_kept_kernel(const char* x, unsigned char* x8, float* scales, int L,
                                                            int d, int block, int nblk) {
    const int b = blockIdx.x, bh = blockIdx.y;
    const int r0 = b * block, r1 = min(r0 + block, L);
    const long long e0 = ((long long)bh * L + r0) * d;
    const int n8 = (r1 - r0) * d / 8;                     // <= 256 * kKeep, checked by the host
    const char* src = x + e0 * 2;
    unsigned char* dst = x8 + e0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    u32x4 held[kKeep];
#pragma unroll
    for (int p = 0; p < kKeep; ++p) {
        const int i = tid + 256 * p;
        held[p] = i < n8 ? ld16_streamed(src + (long long)i * 16) : u32x4{0, 0, 0, 0};
    }
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < kKeep; ++p) amax = fmaxf(amax, piece_amax<T>(held[p]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float red[4];
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
    if (tid == 0) scales[(long long)bh * nblk + b] = s;
#pragma unroll
    for (int p = 0; p < kKeep; ++p) {
        const int i = tid + 256 * p;
        if (i < n8) quant_store<T>(held[p], s, dst + (long long)i * 8);
    }
}

// Larger blocks: one pass for the maximum, a second that reads and converts.
template <class T>
__global__ __launch_bounds__(256) void fa_quant_streamed_kernel(const char* x, unsigned char* x8, float* scales,
                                                                int L, int d, int block, int nblk) {
    const int b = blockIdx.x, bh = blockIdx.y;
    const int r0 = b * block, r1 = min(r0 + block, L);
    const long long e0 = ((long long)bh * L + r0) * d;
    const long long n8 = (long long)(r1 - r0) * d / 8;   // 16-byte input pieces of the block
    const char* src = x + e0 * 2;
    unsigned char* dst = x8 + e0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    float amax = 0.f;
    // the first pass leaves the block in the caches for the second
    for (long long i = tid; i < n8; i += 256) amax = fmaxf(amax, piece_amax<T>(ld16(src + i * 16)));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float red[4];
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
    if (tid == 0) scales[(long long)bh * nblk + b] = s;
    for (long long i = tid; i < n8; i += 256) quant_store<T>(ld16_streamed(src + i * 16), s, dst + i * 8);
}

template <class T>
int launch_quant(const void* x, void* x8, float* scales, int L, int d, int block, int nblk, dim3 grid,
                 hipStream_t stream) {
    const bool kept = (long long)block * d / 8 <= 256 * kKeep;
    return fa_detail::launch_kernel(kept ? fa_quant_kept_kernel<T> : fa_quant_streamed_kernel<T>, grid, dim3(256),
                                    stream, static_cast<const char*>(x), static_cast<unsigned char*>(x8), scales, L,
                                    d, block, nblk);
}

}  // namespace

extern "C" int fa_quantize_fp8(const void* x, int dtype, int B, int H, int L, int d, int block, void* x8,
                               float* scales, hipStream_t stream) {
    if (!x || !x8 || !scales) return FA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || L <= 0 || block < 1) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H > 65535) return FA_ERR_INVALID_ARG;
    // one head's tensor must stay below 2 GiB, as for fa_fwd
    if ((long long)L * d * 2 >= (1LL << 31)) return FA_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)x8) % 16 != 0 || (uintptr_t)scales % 4 != 0) return FA_ERR_ALIGN;
    const long long nblk = ((long long)L + block - 1) / block;     // <= L
    const dim3 grid((unsigned)nblk, (unsigned)(B * H));
    if (dtype == FA_BF16) return launch_quant<__bf16>(x, x8, scales, L, d, block, (int)nblk, grid, stream);
    return launch_quant<_Float16>(x, x8, scales, L, d, block, (int)nblk, grid, stream);
}
