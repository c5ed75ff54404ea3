// Split-K/V attention for a few query rows against a long K/V sequence
// (decoding), for gfx950.
//
// Flash-Decoding ("04 Transformers, Attention, and FlashAttention", the
// Flash Decoding steps): the keys of each (batch, head) are cut into nsplit
// contiguous chunks; each chunk is attended to on its own, exactly as one
// FlashAttention task, giving a normalised partial output O_s and its
// logsumexp lse_s; a second kernel merges the chunks with the rescale rule of
// the online softmax ("FlashAttention 深度解析", first article: statistics are
// brought to a common maximum by exp(m_old - m_new) and added):
//     lse = ln sum_s exp(lse_s),    O = sum_s exp(lse_s - lse) O_s.
//
// This work reads every K/V byte once and does about one flop per byte, so it
// is bound by HBM bandwidth, not by the matrix cores: the kernels use plain
// vector FMA and put their effort into coalesced 16-byte loads with many of
// them in flight.
//
// gfx950 mapping of fa_splitkv_kernel: one wavefront per chunk; a key row of
// d elements is spread over 16 lanes (d/16 elements each, 16 bytes at
// d = 128 in 16-bit types), so one wave load covers 4 consecutive key rows
// (1 KB, fully coalesced).  A lane keeps the d/16 query elements of every
// query row and the matching slice of the running output.  Per block of 4U
// keys: the 16-lane partial dot products are summed with lane exchanges, the
// block maximum of each query row is taken across the wave, the running sum
// and output are rescaled, and exp2 weights update both.  The four 4-key
// lane groups share the running maximum, so at the end only their sums and
// outputs are added (two exchanges).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace {

using namespace fa_dev;

constexpr int kMaxLq = 8;

// K and V are read once per call, so their loads carry the nontemporal hint:
// the lines stream through the caches without displacing anything (on the
// decode shape 5.79 -> 6.60 TB/s, results bitwise equal).
template <class T, int E>
__device__ inline void load_elems_streamed(const char* p, float* out) {
    constexpr int BYTES = E * (int)sizeof(T);
    if constexpr (BYTES % 16 == 0) {
        u32x4 r[BYTES / 16];
#pragma unroll
        for (int c = 0; c < BYTES / 16; ++c) r[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + c);
        load_elems<T, E>(reinterpret_cast<const char*>(r), out);
    } else {
        static_assert(BYTES == 8, "8 or a multiple of 16 bytes per lane");
        const u32x2 r = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        load_elems<T, E>(reinterpret_cast<const char*>(&r), out);
    }
}

struct SkParams {
    const char* q;      // (BH, Lq, D)
    const char* k;      // (BH, Lk, D)
    const char* v;
    float* opart;       // (nsplit, BH, Lq, D) normalised partial outputs
    float* lpart;       // (nsplit, BH, Lq) partial logsumexp
    int BH, Lq, Lk, nsplit, chunk;
    float c;            // scale * log2(e): scores in base-2 exponent units
};

// Keys per lane per block: bounded by registers (LQ scores per key).
template <int LQ>
struct SkShape {
    static constexpr int U = LQ == 1 ? 16 : (LQ == 2 ? 8 : (LQ == 4 ? 4 : 2));
};

template <class T, int D, int LQ>
__global__ __launch_bounds__(256) void fa_splitkv_kernel(SkParams p) {
    constexpr int E = D / 16;                 // row elements per lane
    constexpr int U = SkShape<LQ>::U;
    constexpr int ES = (int)sizeof(T);
    const int lane = threadIdx.x & 63;
    const int split = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (split >= p.nsplit) return;            // whole waves only; this kernel has no barrier
    const int bh = blockIdx.y;
    const int ds = lane & 15;                 // which d/16 slice of a row
    const int kg = lane >> 4;                 // which of 4 consecutive keys
    const int k0 = split * p.chunk;
    const int k1 = min(k0 + p.chunk, p.Lk);

    // query slices, scaled into base-2 exponent units
    float qv[LQ][E];
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
        if (i < p.Lq) {
            load_elems<T, E>(p.q + (((long long)bh * p.Lq + i) * D + ds * E) * ES, qv[i]);
#pragma unroll
            for (int e = 0; e < E; ++e) qv[i][e] *= p.c;
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) qv[i][e] = 0.f;
        }
    }
    float m[LQ], l[LQ], o[LQ][E];
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[i][e] = 0.f;
    }

    const char* kh = p.k + (long long)bh * p.Lk * D * ES + ds * E * ES;
    const char* vh = p.v + (long long)bh * p.Lk * D * ES + ds * E * ES;
    for (int kb = k0; kb < k1; kb += 4 * U) {
        float kr[U][E], vr[U][E];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int key = kb + 4 * u + kg;
            valid[u] = key < k1;
            const long long row = valid[u] ? key : k1 - 1;      // in range; masked below
            load_elems_streamed<T, E>(kh + row * D * ES, kr[u]);
            load_elems_streamed<T, E>(vh + row * D * ES, vr[u]);
        }
        float s[U][LQ];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < LQ; ++i) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) dot = __builtin_fmaf(qv[i][e], kr[u][e], dot);
                // sum over the 16 lanes holding this key's row
                dot += __shfl_xor(dot, 1);
                dot += __shfl_xor(dot, 2);
                dot += __shfl_xor(dot, 4);
                dot += __shfl_xor(dot, 8);
                s[u][i] = valid[u] ? dot : -INFINITY;
            }
#pragma unroll
        for (int i = 0; i < LQ; ++i) {
            float mb = s[0][i];
#pragma unroll
            for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][i]);
            mb = fmaxf(mb, __shfl_xor(mb, 16));
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float m_new = fmaxf(m[i], mb);
            if (m_new > m[i]) {                       // wave-uniform per query row
                const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);   // 0 while m was -inf
                l[i] *= alpha;
#pragma unroll
                for (int e = 0; e < E; ++e) o[i][e] *= alpha;
                m[i] = m_new;
            }
            const float ref = m[i] == -INFINITY ? 0.f : m[i];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float pu = __builtin_amdgcn_exp2f(s[u][i] - ref);     // 0 for masked keys
                l[i] += pu;
#pragma unroll
                for (int e = 0; e < E; ++e) o[i][e] = __builtin_fmaf(pu, valid[u] ? vr[u][e] : 0.f, o[i][e]);
            }
        }
    }

    // add the four key groups' sums and outputs (the maximum is shared)
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
        l[i] += __shfl_xor(l[i], 16);
        l[i] += __shfl_xor(l[i], 32);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            o[i][e] += __shfl_xor(o[i][e], 16);
            o[i][e] += __shfl_xor(o[i][e], 32);
        }
    }
    if (kg == 0) {
#pragma unroll
        for (int i = 0; i < LQ; ++i) {
            if (i >= p.Lq) break;
            const long long row = ((long long)split * p.BH + bh) * p.Lq + i;
            const bool any = l[i] > 0.f;                 // false for an empty chunk
            const float inv = any ? 1.f / l[i] : 0.f;
            float* od = p.opart + row * D + ds * E;
#pragma unroll
            for (int e = 0; e < E; ++e) od[e] = o[i][e] * inv;
            if (ds == 0) p.lpart[row] = any ? (m[i] + __builtin_amdgcn_logf(l[i])) * kLn2 : -INFINITY;
        }
    }
}

// One wavefront per output row (b, h, query): merge the nsplit partials.
template <class T, int D>
__global__ __launch_bounds__(256) void fa_combine_kernel(const float* opart, const float* lpart, T* o, float* lse,
                                                         int nsplit, long long rows) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    constexpr int PER = D / 64;               // output elements per lane
    float mx = -INFINITY;
    for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, lpart[(long long)s * rows + row]);
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) mx = fmaxf(mx, __shfl_xor(mx, w));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float total = -INFINITY;
    if (mx != -INFINITY) {
        float wsum = 0.f;
        for (int s = lane; s < nsplit; s += 64)
            wsum += __builtin_amdgcn_exp2f((lpart[(long long)s * rows + row] - mx) * kLog2e);
#pragma unroll
        for (int w = 1; w < 64; w <<= 1) wsum += __shfl_xor(wsum, w);
        total = mx + __builtin_amdgcn_logf(wsum) * kLn2;
        for (int s = 0; s < nsplit; ++s) {
            const float ls = lpart[(long long)s * rows + row];
            const float w = __builtin_amdgcn_exp2f((ls - total) * kLog2e);   // 0 for an empty partial
            const float* op = opart + ((long long)s * rows + row) * D;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(w, op[lane + 64 * e], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) o[row * D + lane + 64 * e] = (T)acc[e];
    if (lane == 0) lse[row] = total;
}

// ---- host side ----

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Chunks per (batch, head) when the caller passes nsplit <= 0: about 2048
// wavefronts in all (two per SIMD), each streaming one long chunk, at least
// 256 keys each.  Above 4 the count is a multiple of 4, so every workgroup's
// four waves have a chunk.  Measured on decoding shapes (Lq 1 to 4, B*H 32 to
// 512, Lk 8K to 64K): fewer, longer streams read HBM faster than the 4096
// shorter ones this rule replaced, by up to 12%; at Lq <= 2 about 1024 waves
// read faster still, at Lq = 4 they fall behind.
int auto_splits(int B, int H, int Lk) {
    const long long bh = (long long)B * H;
    long long want = (2048 + bh - 1) / bh;
    if (want > 4) want = (want + 3) / 4 * 4;
    const long long cap = ((long long)Lk + 255) / 256;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return (int)want;
}

size_t workspace_bytes(long long rows, int d, int nsplit) {
    // partial outputs, then partial lse, each 256-byte aligned
    const size_t ob = ((size_t)nsplit * rows * d * sizeof(float) + 255) / 256 * 256;
    const size_t lb = ((size_t)nsplit * rows * sizeof(float) + 255) / 256 * 256;
    return ob + lb;
}

template <class T, int D, int LQ>
int launch_split(const SkParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((p.nsplit + 3) / 4), (unsigned)p.BH);
    return fa_detail::launch_kernel(fa_splitkv_kernel<T, D, LQ>, grid, dim3(256), stream, p);
}

template <class T, int D>
int launch_split_lq(const SkParams& p, hipStream_t stream) {
    if (p.Lq == 1) return launch_split<T, D, 1>(p, stream);
    if (p.Lq == 2) return launch_split<T, D, 2>(p, stream);
    if (p.Lq <= 4) return launch_split<T, D, 4>(p, stream);
    return launch_split<T, D, 8>(p, stream);
}

template <class T, int D>
int launch_combine(const float* opart, const float* lpart, void* o, float* lse, int nsplit, long long rows,
                   hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    return fa_detail::launch_kernel(fa_combine_kernel<T, D>, grid, dim3(256), stream, opart, lpart, static_cast<T*>(o),
                                    lse, nsplit, rows);
}

int dispatch_combine(const float* opart, const float* lpart, void* o, float* lse, int nsplit, long long rows, int d,
                     int dtype, hipStream_t stream) {
    if (dtype == FA_BF16)
        return d == 64 ? launch_combine<__bf16, 64>(opart, lpart, o, lse, nsplit, rows, stream)
                       : launch_combine<__bf16, 128>(opart, lpart, o, lse, nsplit, rows, stream);
    if (dtype == FA_F16)
        return d == 64 ? launch_combine<_Float16, 64>(opart, lpart, o, lse, nsplit, rows, stream)
                       : launch_combine<_Float16, 128>(opart, lpart, o, lse, nsplit, rows, stream);
    return d == 64 ? launch_combine<float, 64>(opart, lpart, o, lse, nsplit, rows, stream)
                   : launch_combine<float, 128>(opart, lpart, o, lse, nsplit, rows, stream);
}

// Checks shared by both entry points.  Grid limit: rows / 4 blocks for the
// combine, 65535 (b, h) pairs per split launch.
int check_common(int B, int H, int Lq, int d, int dtype) {
    if (B <= 0 || H <= 0 || Lq <= 0) return FA_ERR_INVALID_ARG;
    if ((long long)B * H > 65535) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// Checks of fa_fwd_splitkv's arguments other than the workspace; fills
// nsplit (automatic when <= 0) and the partial-result row count.
int check_splitkv(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int Lq,
                  int Lk, int d, float scale, int dtype, int& nsplit, long long& rows) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    int rc = check_common(B, H, Lq, d, dtype);
    if (rc != FA_OK) return rc;
    // Lk up to 2^30 keeps the chunk bounds (split * chunk, key + 64) inside int
    if (Lk <= 0 || Lk > (1 << 30)) return FA_ERR_INVALID_ARG;
    if (Lq > kMaxLq) return FA_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if ((long double)B * H * Lk * d >= 4.6e18L) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    if (nsplit <= 0) nsplit = auto_splits(B, H, Lk);
    if (nsplit > 4 * 65535) return FA_ERR_INVALID_ARG;
    rows = (long long)B * H * Lq;
    return FA_OK;
}

// The chunk kernel into the partial results at `workspace` (256-byte
// aligned, workspace_bytes(rows, d, nsplit) long), then the merge.
int run_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq, int Lk,
                int d, float scale, int dtype, int nsplit, long long rows, void* workspace, hipStream_t stream) {
    float* opart = static_cast<float*>(workspace);
    float* lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            ((size_t)nsplit * rows * d * sizeof(float) + 255) / 256 * 256);
    SkParams p;
    p.q = static_cast<const char*>(q);
    p.k = static_cast<const char*>(k);
    p.v = static_cast<const char*>(v);
    p.opart = opart;
    p.lpart = lpart;
    p.BH = B * H;
    p.Lq = Lq;
    p.Lk = Lk;
    p.nsplit = nsplit;
    p.chunk = (Lk + nsplit - 1) / nsplit;
    p.c = scale * kLog2e;

    int rc;
    if (dtype == FA_BF16)
        rc = d == 64 ? launch_split_lq<__bf16, 64>(p, stream) : launch_split_lq<__bf16, 128>(p, stream);
    else if (dtype == FA_F16)
        rc = d == 64 ? launch_split_lq<_Float16, 64>(p, stream) : launch_split_lq<_Float16, 128>(p, stream);
    else
        rc = d == 64 ? launch_split_lq<float, 64>(p, stream) : launch_split_lq<float, 128>(p, stream);
    if (rc != FA_OK) return rc;
    return dispatch_combine(opart, lpart, o, lse, nsplit, rows, d, dtype, stream);
}

// ---- the library's own scratch for fa_fwd_splitkv_noalloc ----
//
// One array per GPU, allocated with the code object when the library is first
// used on that GPU and held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the device
// address that hipGetSymbolAddress returns for the current device, looked up
// once per device and kept in g_scratch.
constexpr int kMaxDevices = 64;
static __device__ __attribute__((aligned(256))) char scratch[FA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of `scratch` on `dev`, with `dev` made current for the
// lookup (and the caller's current device restored).
int scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = -1;
        hipError_t err = hipGetDevice(&cur);
        if (err != hipSuccess) return fa_detail::status_of(err);
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return fa_detail::status_of(err);
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return fa_detail::status_of(err);
        if (ptr == nullptr || (uintptr_t)ptr % 256 != 0) return fa_detail::status_of(hipErrorInvalidSymbol);
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return FA_OK;
}

}  // namespace

extern "C" size_t fa_splitkv_workspace_bytes(int B, int H, int Lq, int Lk, int d, int nsplit) {
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || (d != 64 && d != 128)) return 0;
    if (nsplit <= 0) nsplit = auto_splits(B, H, Lk);
    return workspace_bytes((long long)B * H * Lq, d, nsplit);
}

extern "C" int fa_splitkv_splits(int B, int H, int Lk) {
    if (B <= 0 || H <= 0 || Lk <= 0) return 0;
    return auto_splits(B, H, Lk);
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lq,
                              int Lk, int d, float scale, int dtype, int nsplit, void* workspace,
                              size_t workspace_size, hipStream_t stream) {
    long long rows = 0;
    const int rc = check_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, rows);
    if (rc != FA_OK) return rc;
    if (!workspace) return FA_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
    if (workspace_size < workspace_bytes(rows, d, nsplit)) return FA_ERR_INVALID_ARG;
    return run_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, rows, workspace, stream);
}

extern "C" int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                      int Lq, int Lk, int d, float scale, int dtype, int nsplit, hipStream_t stream) {
    long long rows = 0;
    int rc = check_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, rows);
    if (rc != FA_OK) return rc;
    if (workspace_bytes(rows, d, nsplit) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    // the GPU the work runs on: the stream's, or the current one for the null stream
    int dev = -1;
    const hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) return fa_detail::status_of(err);
    void* ws = nullptr;
    rc = scratch_on(dev, &ws);
    if (rc != FA_OK) return rc;
    return run_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, scale, dtype, nsplit, rows, ws, stream);
}

extern "C" int fa_combine(const float* o_part, const float* lse_part, int nsplit, int B, int H, int Lq, int d,
                          void* o, float* lse, int dtype, hipStream_t stream) {
    if (!o_part || !lse_part || !o || !lse) return FA_ERR_INVALID_ARG;
    int rc = check_common(B, H, Lq, d, dtype);
    if (rc != FA_OK) return rc;
    if (nsplit <= 0) return FA_ERR_INVALID_ARG;
    const long long rows = (long long)B * H * Lq;
    if ((rows + 3) / 4 > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
    if (!aligned(o_part, 4) || !aligned(lse_part, 4) || !aligned(o, 16) || !aligned(lse, 4)) return FA_ERR_ALIGN;
    return dispatch_combine(o_part, lse_part, o, lse, nsplit, rows, d, dtype, stream);
}
