// Device building blocks shared by the library's gfx950 kernels (not part of
// the C ABI): fragment types, the 32x32 MFMA step per storage type, 16-byte
// accesses, the LDS row swizzle, buffer descriptors and the LDS-DMA load.
#ifndef FA_DEVICE_H
#define FA_DEVICE_H

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace fa_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- per storage type: fragment of 8 k-values per lane, and the MFMA step ----
template <class T>
struct Ty;

template <>
struct Ty<__bf16> {
    using frag = bf16x8;
    static constexpr int kBytes = 2;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag cvt(const float* x) {
        frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
        return r;
    }
};

template <>
struct Ty<_Float16> {
    using frag = f16x8;
    static constexpr int kBytes = 2;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag cvt(const float* x) {
        frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[e];
        return r;
    }
};

template <>
struct Ty<float> {
    using frag = f32x8;
    static constexpr int kBytes = 4;
    // eight k=2 steps; element e of every lane's fragment feeds step e, so
    // both operands see the same k order
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
    __device__ static inline frag cvt(const float* x) {
        frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = x[e];
        return r;
    }
};

// 16-byte global / LDS accesses
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }
__device__ inline void st8(void* p, u32x2 x) { *reinterpret_cast<u32x2*>(p) = x; }

// LDS row layout of a K or V tile in the 16-bit kernels: unpadded rows of D
// elements; 16-byte chunk c of row r is stored at chunk c ^ f(r).  fk spreads
// the same chunk of 16 consecutive rows over 16 bank slots (row reads); fv
// spreads a 64-byte column band of 4 consecutive rows (transposing reads).
template <int D>
struct HLayout {
    static constexpr int P = D * 2;       // row pitch in LDS (bytes), unpadded
    static constexpr int CPR = D / 8;     // 16-byte chunks per row
    __device__ static inline int fk(int r) { return (CPR == 16 ? r : (r >> 1)) & (CPR - 1); }
    __device__ static inline int fv(int r) { return 4 * ((CPR == 16 ? r : (r >> 1)) & (CPR / 4 - 1)); }
};

// buffer descriptor word 3 for CDNA: raw, untyped 32-bit access
constexpr int kBufWord3 = 0x00020000;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes): reads past the end return 0.
__device__ inline i32x4 buffer_rsrc(const void* base, int bytes) {
    const unsigned long long b = (unsigned long long)base;
    i32x4 r;
    r[0] = (int)(b & 0xffffffffu);
    r[1] = (int)(b >> 32);   // stride 0
    r[2] = bytes;
    r[3] = kBufWord3;
    return r;
}

// The same buffer advanced by `off` bytes (off a multiple of 16): offsets
// are checked against what is left, so reads past the end still return 0.
__device__ inline i32x4 buffer_rsrc_at(const char* base, int bytes, int off) {
    return buffer_rsrc(base + off, max(bytes - off, 0));
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_base + 16*lane
// (buffer_load_dwordx4 ... lds).  Issued as inline asm so that the compiler's
// wait-count insertion does not make later LDS reads wait for this DMA: the
// kernel waits for it explicitly (vmcnt) before the barrier that publishes the
// tile.  M0 carries the LDS address and is restored afterwards.
__device__ inline void dma16(i32x4 rsrc, int voff, unsigned lds_base) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(voff), "s"(rsrc)
        : "memory");
}

// Row stores from a transposed 32x32 accumulator: for the row it owns, a
// lane of half h holds columns 8c + 4h .. 8c + 4h + 3 of every 8-column chunk
// c, and lane^32 holds the other four.  One exchange of 8 bytes per pair of
// chunks (c0, c0 + 1) lets the lower lane store chunk c0 and the upper lane
// chunk c0 + 1 as one 16-byte store each, instead of two 8-byte stores per
// lane.  `lo` and `hi` are this lane's halves of chunks c0 and c0 + 1; both
// lanes of the pair must call it (they share the row).  The exchange is
// v_permlane32_swap of (lo, hi): it trades the upper lanes' lo with the lower
// lanes' hi, which leaves the lower lane holding both halves of chunk c0 and
// the upper lane both halves of chunk c0 + 1, each in order.
template <class T>
__device__ inline void store_chunk_pair(char* row, int c0, int h, const T (&lo)[4], const T (&hi)[4]) {
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    const auto s0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
    st16(row + (c0 + h) * 8 * (int)sizeof(T), u32x4{s0[0], s1[0], s0[1], s1[1]});
}

// Exchange with lane^32 (v_permlane32_swap): returns the pair {x, x of lane^32}.
__device__ inline float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// E consecutive elements of a row, widened to fp32 (E = 4 or 8).
template <class T, int E>
__device__ inline void load_elems(const char* p, float* out);

template <>
__device__ inline void load_elems<__bf16, 8>(const char* p, float* out) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[2 * j] = __uint_as_float(r[j] << 16);
        out[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
}
template <>
__device__ inline void load_elems<__bf16, 4>(const char* p, float* out) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        out[2 * j] = __uint_as_float(r[j] << 16);
        out[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
}
// The two binary16 halves of a 32-bit word.  (Scalar bit casts: a bit cast
// of a vector element to a two-half vector was compiled into a load of only
// the first word.)
__device__ inline void halves(unsigned w, float* out) {
    out[0] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
    out[1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
template <>
__device__ inline void load_elems<_Float16, 8>(const char* p, float* out) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
    halves(r[0], out);
    halves(r[1], out + 2);
    halves(r[2], out + 4);
    halves(r[3], out + 6);
}
template <>
__device__ inline void load_elems<_Float16, 4>(const char* p, float* out) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(p);
    halves(r[0], out);
    halves(r[1], out + 2);
}
template <>
__device__ inline void load_elems<float, 8>(const char* p, float* out) {
    const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
    const u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[j] = __uint_as_float(a[j]);
        out[4 + j] = __uint_as_float(b[j]);
    }
}
template <>
__device__ inline void load_elems<float, 4>(const char* p, float* out) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(a[j]);
}

}  // namespace fa_dev

#endif
