// Backward pass of exact attention for gfx950 (MI355X), 16-bit types.
//
// Gradients for an upstream dO ("FlashAttention 深度解析", first article,
// section 4: dV = P^T dO, dP = dO V^T, dS = dP (.) P - P (.) rowsum(dP (.) P),
// and the chain rule through S = scale Q K^T for dQ and dK), with P
// recomputed from Q, K and the logsumexp the forward pass stored instead of
// being kept ("Recomputation": "04 Transformers, Attention, and
// FlashAttention" and "FlashAttention: как реально считается attention на
// GPU", backward pass).  rowsum(dP (.) P)_i equals dO_i . O_i, because
// O_i = sum_j P_ij V_j; a first kernel computes that vector D from O.
//
// gfx950 mapping.  Two kernels do the matrix work, neither needs atomics:
//  * fa_bwd_dkdv_kernel: one workgroup per 128 keys of a head (4 waves x 32
//    keys; K and V rows of a wave live in registers as MFMA B operands).  It
//    streams the head's Q and dO in 64-row tiles through LDS and, per 32x32
//    block, computes S = Q K^T and dP = dO V^T (lane = key: the accumulator
//    column), P and dS with each query row's lse and D read from LDS, and
//    accumulates dV^T += dO^T P and dK^T += Q^T dS, the dO^T and Q^T operands
//    coming from transposing LDS reads.
//  * fa_bwd_dq_kernel: one workgroup per 128 queries (4 waves x 32 queries;
//    Q and dO rows in registers).  It streams K and V in 64-row tiles and
//    computes S^T = K Q^T and dP^T = V dO^T (lane = query, so lse and D are
//    one value per lane), dS^T, and dQ^T += K^T dS^T.
//  So dK/dV and dQ are each reduced inside one workgroup; the price is that
//  S and dP are formed twice (seven 32x32-tile products per block instead of
//  five).  Tiles arrive by LDS-DMA into double-buffered stages, rows
//  XOR-swizzled so that both the row reads and the transposing reads are
//  free of bank conflicts.  Both kernels run a 1-D grid: heads grouped per
//  XCD, and causal blocks in heavy-first order across all heads.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace {

using namespace fa_dev;

struct BwdParams {
    const char* q;
    const char* k;
    const char* v;
    const char* o;
    const char* dout;
    const float* lse;       // (BH, L) natural-log logsumexp from the forward pass
    float* dvec;            // (BH, L) D_i = dO_i . O_i (workspace)
    char* dq;
    char* dk;
    char* dv;
    int BH, L;
    float c;                // scale * log2(e)
    float scale;
};

// Streamed tiles: 64 rows of D elements, 16-bit.
template <int D>
struct BCfg {
    static constexpr int P = 2 * D;               // LDS row pitch (bytes)
    static constexpr int ROWS = 64;
    static constexpr int TILE = ROWS * P;
    static constexpr int PPW = TILE / 1024 / 4;   // 1 KB DMA pieces per wave per tile
    static_assert(PPW * 4 * 1024 == TILE, "tile must split into 1 KB pieces");
};

// ---- D_i = dO_i . O_i: 16 lanes per row ----
template <class T, int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(BwdParams p, long long rows) {
    constexpr int E = D / 16;
    const int lane = threadIdx.x & 63;
    const long long row = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const bool valid = row < rows;
    float acc = 0.f;
    if (valid) {
        float g[E], o[E];
        const long long off = (row * D + (lane & 15) * E) * 2;
        load_elems<T, E>(p.dout + off, g);
        load_elems<T, E>(p.o + off, o);
#pragma unroll
        for (int e = 0; e < E; ++e) acc = __builtin_fmaf(g[e], o[e], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 8);
    if (valid && (lane & 15) == 0) p.dvec[row] = acc;
}

// Row layout of the streamed tiles.  Each tile is read two ways: as rows
// (16 lanes of a ds_read_b128 pass read one chunk of 16 different rows) and
// transposed (32 lanes of a ds_read_b64_tr_b16 pass read 4 consecutive rows,
// 4 chunks each).  Chunk c of row r is stored at c ^ fb(r): fb is a bijection
// on the 16 rows that share a bank position (row reads conflict-free), and
// its bit 2 and up (which 4-chunk group a row's chunks land in) differs
// between the rows of one 4-row step that share a bank position (transposing
// reads conflict-free).  d = 128 (rows of 256 bytes, all rows at bank 0):
// fb = 4 (r mod 4) + (r / 4 mod 4).  d = 64 (two rows per 256 bytes):
// fb = 4 (r / 2 mod 2) + (r / 4 mod 4).
template <int D>
__device__ inline int fb(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Per-lane LDS offsets shared by both kernels, all derived from two base
// values by XOR with constants (so only the bases stay live across a loop).
//  row(s)    : the 16-byte chunk (2s + hf) of row l32 (A operand of a row
//              product: lane = row, 8 consecutive d).  That chunk sits at
//              (2s + hf) ^ fk(l32); s only enters the bits above bit 0 of the
//              chunk index, so row(s) = row(0) ^ (s << 5).
//  tr(dt,hi) : transposing reads (A operand d x rows): lane 16g+4e+q reads
//              row 4*(g>>1) + e (+8 for hi) of a 16-row step, d columns of
//              chunk 4dt + 2(g&1) + (q>>1), half (q&1).  dt flips chunk bits
//              2.. (offset bits 6..); the +8 rows flip one row bit and fb's
//              bit 1.  Rows 0..15 and 16..31 of a 32-row group share the
//              swizzle (period 16).
template <int D>
struct Offs {
    static constexpr int kTrHi = D == 128 ? 0x820 : 0x420;
    int row0, tr0;
    __device__ int row(int s) const { return row0 ^ (s << 5); }
    __device__ int tr(int dt, int hi) const { return tr0 ^ (dt << 6) ^ (hi ? kTrHi : 0); }
    __device__ void init(int lane) {
        constexpr int P = 2 * D;
        const int l32 = lane & 31, hf = lane >> 5;
        row0 = l32 * P + ((hf ^ fb<D>(l32)) << 4);
        const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
        const int r = 4 * (g >> 1) + e;
        const int c = 2 * (g & 1) + (q >> 1);
        tr0 = r * P + ((c ^ fb<D>(r)) << 4) + 8 * (q & 1);
    }
    // The same offsets, opaque to the optimiser: called inside a loop body, the
    // derived offsets are recomputed there (a few XORs) instead of being
    // hoisted and kept live, or spilled, across the loop.
    __device__ Offs fresh() const {
        Offs o = *this;
        asm volatile("" : "+v"(o.row0), "+v"(o.tr0));
        return o;
    }
};

// DMA: piece n of a tile (1 KB, lane l its 16 bytes at LDS offset 1024n+16l)
// holds global chunk slot ^ fb(row) of that row.  For the PPW pieces of one
// wave, piece wave*PPW + x reads at dma_goff(wave*PPW) ^ (x * kPieceX): x
// adds 1024 bytes of rows (bit 10 up) and flips fb bits the piece's rows
// determine (chunk bit 0 at d = 128, bit 1 at d = 64).
template <int D>
constexpr int kPieceX = D == 128 ? 0x410 : 0x420;

template <int D>
__device__ inline int dma_goff(int n, int lane) {
    constexpr int P = 2 * D;
    const int o = 1024 * n + 16 * lane;
    const int r = o / P, slot = (o % P) >> 4;
    return r * P + ((slot ^ fb<D>(r)) << 4);
}

// A operand read transposed from a row-major tile at row offset rowb (bytes).
template <class T>
__device__ inline typename Ty<T>::frag tr_frag(const lds_char* base, int lo, int hi) {
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + lo));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + hi));
    return __builtin_bit_cast(typename Ty<T>::frag, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row fragments (lane = row l32 of `rows`, d elements 16s + 8hf .. +7) from
// global memory; zero for rows >= L.
template <class T, int D>
__device__ inline void load_row_frags(const char* base, int row, int L, int hf, typename Ty<T>::frag* f) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4 raw = u32x4{0, 0, 0, 0};
        if (row < L) raw = ld16(base + ((long long)row * D + 16 * s + 8 * hf) * 2);
        f[s] = __builtin_bit_cast(typename Ty<T>::frag, raw);
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(f[s]));
}

// Which (head, block of 128 rows) workgroup blockIdx.x owns, in a 1-D grid
// of BH * nblk.  Workgroup ids are dealt round-robin to the 8 XCDs (id % 8);
// when BH is a multiple of 8 each XCD gets whole heads, whose streamed tiles
// then come through its own L2.  Causal: the blocks with the most work are
// dispatched first, across all heads (heavy_last: the last block is the
// heaviest, else the first).
__device__ inline void bwd_tile(int nblk, int BH, bool causal, bool heavy_last, int& bh, int& blk) {
    const int id = blockIdx.x;
    int rank;                                    // position in dispatch order within the XCD's share
    if (BH % 8 == 0) {
        const int xcd = id & 7, s = id >> 3, hp = BH >> 3;
        if (causal) {
            rank = s / hp;
            bh = xcd * hp + s % hp;
        } else {
            bh = xcd * hp + s / nblk;
            rank = s % nblk;
        }
    } else if (causal) {
        rank = id / BH;
        bh = id % BH;
    } else {
        bh = id / nblk;
        rank = id % nblk;
    }
    blk = causal && heavy_last ? nblk - 1 - rank : rank;
}

// ---- dQ: one workgroup per 128 queries ----
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(BwdParams p) {
    using Cf = BCfg<D>;
    using frag = typename Ty<T>::frag;
    constexpr int P = Cf::P, TILE = Cf::TILE, PPW = Cf::PPW;
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];   // K0 K1 V0 V1

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int L = p.L;
    // causal: the last query blocks see the most keys; dispatch them first
    int bh, qb;
    bwd_tile((L + 127) / 128, p.BH, CAUSAL, true, bh, qb);
    const int q0 = qb * 128;
    const int qw = q0 + 32 * wave;
    const int qend = min(q0 + 128, L);
    const int ntiles = CAUSAL ? (qend + 63) / 64 : (L + 63) / 64;
    const int ntw = qw >= L ? 0 : (CAUSAL ? (min(qw + 32, L) + 63) / 64 : ntiles);
    const long long head = (long long)bh * L * D;
    const char* kh = p.k + head * 2;
    const char* vh = p.v + head * 2;

    const int query = qw + l32;
    frag qf[D / 16], gf[D / 16];
    load_row_frags<T, D>(p.q + head * 2, query, L, hf, qf);
    load_row_frags<T, D>(p.dout + head * 2, query, L, hf, gf);
    const float lse2 = query < L ? p.lse[(long long)bh * L + query] * kLog2e : 0.f;
    const float dval = query < L ? p.dvec[(long long)bh * L + query] : 0.f;
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    Offs<D> off;
    off.init(lane);
    const int goff0 = dma_goff<D>(wave * PPW, lane);
    const unsigned lds0 = (unsigned)(unsigned long long)(lds_char*)smem;
    auto dma_tile = [&](int t) {                  // K_t, V_t into stage t & 1
        const i32x4 kr = buffer_rsrc_at(kh, L * P, t * TILE);
        const i32x4 vr = buffer_rsrc_at(vh, L * P, t * TILE);
        int g0 = goff0;
        asm volatile("" : "+v"(g0));              // derive the piece offsets here, not across the loop
#pragma unroll
        for (int x = 0; x < PPW; ++x) {
            const unsigned dst = lds0 + (t & 1) * TILE + 1024 * (wave * PPW + x);
            dma16(kr, g0 ^ (x * kPieceX<D>), __builtin_amdgcn_readfirstlane(dst));
            dma16(vr, g0 ^ (x * kPieceX<D>), __builtin_amdgcn_readfirstlane(dst + 2 * TILE));
        }
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    auto compute = [&](auto mask_tag, int t) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const char* ks = smem + (t & 1) * TILE;
        const char* vs = smem + 2 * TILE + (t & 1) * TILE;
        const lds_char* ksl = (const lds_char*)smem + (t & 1) * TILE;
        const Offs<D> o = off.fresh();
        const int last = CAUSAL ? min(query, L - 1) : L - 1;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x16 st, dpt;
#pragma unroll
            for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.f;
            // K and V row operands are read two steps ahead of their MFMAs,
            // the transposed K operands of the dQ products likewise
            frag ka3[3], va3[3];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                ka3[s] = __builtin_bit_cast(frag, ld16(ks + kt * 32 * P + o.row(s)));
                va3[s] = __builtin_bit_cast(frag, ld16(vs + kt * 32 * P + o.row(s)));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                if (s + 2 < D / 16) {
                    ka3[(s + 2) % 3] = __builtin_bit_cast(frag, ld16(ks + kt * 32 * P + o.row(s + 2)));
                    va3[(s + 2) % 3] = __builtin_bit_cast(frag, ld16(vs + kt * 32 * P + o.row(s + 2)));
                }
                st = Ty<T>::mma(ka3[s % 3], qf[s], st);
                dpt = Ty<T>::mma(va3[s % 3], gf[s], dpt);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // register r holds key t*64 + 32kt + 4hf + 8(r/4) + r%4
            const int lim = last - t * 64 - 32 * kt - 4 * hf;
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], p.c, -lse2));
                if (MASK && 8 * (r >> 2) + (r & 3) > lim) pr = 0.f;
                ds[r] = pr * (dpt[r] - dval);
            }
            const frag d0 = Ty<T>::cvt(ds), d1 = Ty<T>::cvt(ds + 8);
            constexpr int NI = D / 16;            // (ps, dt) = (i / (D/32), i % (D/32))
            frag ta[3];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                ta[i] = tr_frag<T>(ksl + (kt * 32 + 16 * (i / (D / 32))) * P, o.tr(i % (D / 32), 0),
                                   o.tr(i % (D / 32), 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (i + 2 < NI) {
                    const int j = i + 2;
                    ta[j % 3] = tr_frag<T>(ksl + (kt * 32 + 16 * (j / (D / 32))) * P, o.tr(j % (D / 32), 0),
                                           o.tr(j % (D / 32), 1));
                }
                acc[i % (D / 32)] = Ty<T>::mma(ta[i % 3], i / (D / 32) ? d1 : d0, acc[i % (D / 32)]);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // first tile with keys past this wave's first query or past L; the
    // tiles before it and from it on run in separate loops, so that only one
    // variant of the tile code is live at a time (register budget)
    const int jmask = CAUSAL ? min(qw / 64, (L - 1) / 64) : (L - 1) / 64;
    const int jm = min(jmask, ntiles);
    auto step = [&](auto mask_tag, int t) {
        if (t + 1 < ntiles) dma_tile(t + 1);
        if (t < ntw) compute(mask_tag, t);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    dma_tile(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int t = 0;
    for (; t < jm; ++t) step(no{}, t);
    for (; t < ntiles; ++t) step(yes{}, t);

    if (query < L) {
        char* qrow = p.dq + (head + (long long)query * D) * 2;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                T a4[4], b4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a4[e] = (T)(acc[dt][8 * gp + e] * p.scale);
                    b4[e] = (T)(acc[dt][8 * gp + 4 + e] * p.scale);
                }
                store_chunk_pair<T>(qrow, 4 * dt + 2 * gp, hf, a4, b4);
            }
    }
}

// ---- dK, dV: one workgroup per 128 keys ----
template <class T, int D, bool CAUSAL>
__device__ __attribute__((always_inline)) inline void fa_bwd_dkdv_body(const BwdParams& p) {
    using Cf = BCfg<D>;
    using frag = typename Ty<T>::frag;
    constexpr int P = Cf::P, TILE = Cf::TILE, PPW = Cf::PPW;
    // Q0 Q1 dO0 dO1, then per stage 64 lse*log2e and 64 D values
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE + 2 * 512];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int L = p.L;
    // causal: the first key blocks see the most queries; dispatch them first
    int bh, kb;
    bwd_tile((L + 127) / 128, p.BH, CAUSAL, false, bh, kb);
    const int k0 = kb * 128;
    const int kw = k0 + 32 * wave;
    const int key = kw + l32;
    const long long head = (long long)bh * L * D;
    const char* qh = p.q + head * 2;
    const char* gh = p.dout + head * 2;

    frag kf[D / 16], vf[D / 16];
    load_row_frags<T, D>(p.k + head * 2, key, L, hf, kf);
    load_row_frags<T, D>(p.v + head * 2, key, L, hf, vf);
    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dka[dt][r] = dva[dt][r] = 0.f;

    Offs<D> off;
    off.init(lane);
    const int goff0 = dma_goff<D>(wave * PPW, lane);
    const unsigned lds0 = (unsigned)(unsigned long long)(lds_char*)smem;
    float* stats = reinterpret_cast<float*>(smem + 4 * TILE);
    auto dma_tile = [&](int t) {                  // Q_t, dO_t into stage t & 1
        const i32x4 qr = buffer_rsrc_at(qh, L * P, t * TILE);
        const i32x4 gr = buffer_rsrc_at(gh, L * P, t * TILE);
        int g0 = goff0;
        asm volatile("" : "+v"(g0));              // derive the piece offsets here, not across the loop
#pragma unroll
        for (int x = 0; x < PPW; ++x) {
            const unsigned dst = lds0 + (t & 1) * TILE + 1024 * (wave * PPW + x);
            dma16(qr, g0 ^ (x * kPieceX<D>), __builtin_amdgcn_readfirstlane(dst));
            dma16(gr, g0 ^ (x * kPieceX<D>), __builtin_amdgcn_readfirstlane(dst + 2 * TILE));
        }
    };
    // row statistics of tile t (wave 0): lse in base-2 units (+inf past L, so
    // P = 0 there) and D
    float st_l = 0.f, st_d = 0.f;
    auto stats_load = [&](int t) {
        const int row = t * 64 + lane;
        st_l = row < L ? p.lse[(long long)bh * L + row] * kLog2e : INFINITY;
        st_d = row < L ? p.dvec[(long long)bh * L + row] : 0.f;
    };
    auto stats_store = [&](int t) {
        stats[(t & 1) * 128 + lane] = st_l;
        stats[(t & 1) * 128 + 64 + lane] = st_d;
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    // 32 queries (rows 32*qt.. of tile t) against this wave's 32 keys
    auto compute = [&](auto mask_tag, int t, int qt) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const char* qs = smem + (t & 1) * TILE;
        const char* gs = smem + 2 * TILE + (t & 1) * TILE;
        const lds_char* qsl = (const lds_char*)smem + (t & 1) * TILE;
        const lds_char* gsl = (const lds_char*)smem + 2 * TILE + (t & 1) * TILE;
        const float* sl = stats + (t & 1) * 128 + 32 * qt;
        const Offs<D> o = off.fresh();
        f32x16 st, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = dp[r] = 0.f;
        // Q and dO row operands are read two steps ahead of their MFMAs, the
        // transposed ones of the dV/dK products one step ahead; the scheduling
        // groups keep that order (the registers allow it at two waves per SIMD)
        frag qa3[3], ga3[3];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            qa3[s] = __builtin_bit_cast(frag, ld16(qs + qt * 32 * P + o.row(s)));
            ga3[s] = __builtin_bit_cast(frag, ld16(gs + qt * 32 * P + o.row(s)));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            if (s + 2 < D / 16) {
                qa3[(s + 2) % 3] = __builtin_bit_cast(frag, ld16(qs + qt * 32 * P + o.row(s + 2)));
                ga3[(s + 2) % 3] = __builtin_bit_cast(frag, ld16(gs + qt * 32 * P + o.row(s + 2)));
            }
            st = Ty<T>::mma(qa3[s % 3], kf[s], st);
            dp = Ty<T>::mma(ga3[s % 3], vf[s], dp);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // register r holds query t*64 + 32qt + 8(r/4) + 4hf + r%4 of key `key`.
        // P and dS are formed and consumed in two halves (registers 8ps..8ps+7,
        // queries 16ps..16ps+15), each feeding its dV and dK products at once.
        const int first = t * 64 + 32 * qt + 4 * hf;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            float pr[8], ds[8];
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const int g = 2 * ps + gg;
                const float4 l4 = *reinterpret_cast<const float4*>(sl + 8 * g + 4 * hf);
                const float4 d4 = *reinterpret_cast<const float4*>(sl + 64 + 8 * g + 4 * hf);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float x = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], p.c, -lv[e]));
                    if (MASK && key > first + 8 * g + e) x = 0.f;
                    pr[4 * gg + e] = x;
                    ds[4 * gg + e] = x * (dp[r] - dv[e]);
                }
            }
            const frag pf = Ty<T>::cvt(pr), sf = Ty<T>::cvt(ds);
            const int rowb = (qt * 32 + 16 * ps) * P;
            frag tg[2], tq[2];
            tg[0] = tr_frag<T>(gsl + rowb, o.tr(0, 0), o.tr(0, 1));
            tq[0] = tr_frag<T>(qsl + rowb, o.tr(0, 0), o.tr(0, 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                if (dt + 1 < D / 32) {
                    tg[(dt + 1) & 1] = tr_frag<T>(gsl + rowb, o.tr(dt + 1, 0), o.tr(dt + 1, 1));
                    tq[(dt + 1) & 1] = tr_frag<T>(qsl + rowb, o.tr(dt + 1, 0), o.tr(dt + 1, 1));
                }
                dva[dt] = Ty<T>::mma(tg[dt & 1], pf, dva[dt]);
                dka[dt] = Ty<T>::mma(tq[dt & 1], sf, dka[dt]);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    const int nq = (L + 63) / 64;
    const int t0 = CAUSAL ? k0 / 64 : 0;          // queries before the first key see none of these keys
    dma_tile(t0);
    if (wave == 0) {
        stats_load(t0);
        stats_store(t0);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // causal: the tiles holding the block's diagonal (queries before k0 + 128)
    // need the mask; the rest do not.  Separate loops keep one variant of the
    // tile code live at a time (register budget).
    auto step = [&](auto mask_tag, int t) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const bool more = t + 1 < nq;
        if (more) {
            dma_tile(t + 1);
            if (wave == 0) stats_load(t + 1);
        }
        if (kw < L) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                // every query before every key of this wave: nothing to add
                if (MASK && t * 64 + 32 * qt + 31 < kw) continue;
                compute(mask_tag, t, qt);
            }
        }
        if (more && wave == 0) stats_store(t + 1);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    };
    const int tdiag = CAUSAL ? min(nq, (k0 + 128 + 63) / 64) : t0;
    int t = t0;
    for (; t < tdiag; ++t) step(yes{}, t);
    for (; t < nq; ++t) step(no{}, t);

    if (key < L) {
        char* krow = p.dk + (head + (long long)key * D) * 2;
        char* vrow = p.dv + (head + (long long)key * D) * 2;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                T ka[4], kb4[4], va[4], vb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ka[e] = (T)(dka[dt][8 * gp + e] * p.scale);
                    kb4[e] = (T)(dka[dt][8 * gp + 4 + e] * p.scale);
                    va[e] = (T)dva[dt][8 * gp + e];
                    vb[e] = (T)dva[dt][8 * gp + 4 + e];
                }
                store_chunk_pair<T>(krow, 4 * dt + 2 * gp, hf, ka, kb4);
                store_chunk_pair<T>(vrow, 4 * dt + 2 * gp, hf, va, vb);
            }
    }
}

// Two waves per SIMD (256 registers a lane): with only the offset bases kept
// across the tile loop, both variants fit without spilling inside it.
template <class T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
    fa_bwd_dkdv_body<T, D, CAUSAL>(p);
}

// ---- host side ----

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <class T, int D, bool CAUSAL>
int launch_bwd(const BwdParams& p, hipStream_t stream) {
    const long long rows = (long long)p.BH * p.L;
    int rc = fa_detail::launch_kernel(fa_bwd_pre_kernel<T, D>, dim3((unsigned)((rows + 15) / 16)), dim3(256), stream,
                                      p, rows);
    if (rc != FA_OK) return rc;
    const dim3 grid((unsigned)((long long)p.BH * ((p.L + 127) / 128)));
    rc = fa_detail::launch_kernel(fa_bwd_dq_kernel<T, D, CAUSAL>, grid, dim3(256), stream, p);
    if (rc != FA_OK) return rc;
    return fa_detail::launch_kernel(fa_bwd_dkdv_kernel<T, D, CAUSAL>, grid, dim3(256), stream, p);
}

template <class T>
int launch_bwd_t(const BwdParams& p, int d, int causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_bwd<T, 64, true>(p, stream) : launch_bwd<T, 64, false>(p, stream);
    return causal ? launch_bwd<T, 128, true>(p, stream) : launch_bwd<T, 128, false>(p, stream);
}

size_t dvec_bytes(long long rows) { return ((size_t)rows * sizeof(float) + 255) / 256 * 256; }

}  // namespace

extern "C" size_t fa_bwd_workspace_bytes(int B, int H, int L) {
    if (B <= 0 || H <= 0 || L <= 0) return 0;
    return dvec_bytes((long long)B * H * L);
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, int B, int H, int L, int d, float scale, int causal, int dtype,
                      void* workspace, size_t workspace_size, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || L <= 0) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * (((long long)L + 127) / 128) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;   // one grid dimension
    // per-head byte offsets go through 32-bit buffer descriptors
    if ((long long)L * d * 2 >= (1LL << 31)) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(workspace, 256))
        return FA_ERR_ALIGN;
    if (workspace_size < dvec_bytes((long long)B * H * L)) return FA_ERR_INVALID_ARG;

    BwdParams p;
    p.q = static_cast<const char*>(q);
    p.k = static_cast<const char*>(k);
    p.v = static_cast<const char*>(v);
    p.o = static_cast<const char*>(o);
    p.dout = static_cast<const char*>(dout);
    p.lse = lse;
    p.dvec = static_cast<float*>(workspace);
    p.dq = static_cast<char*>(dq);
    p.dk = static_cast<char*>(dk);
    p.dv = static_cast<char*>(dv);
    p.BH = B * H;
    p.L = L;
    p.c = scale * kLog2e;
    p.scale = scale;
    return dtype == FA_BF16 ? launch_bwd_t<__bf16>(p, d, causal, stream) : launch_bwd_t<_Float16>(p, d, causal, stream);
}
