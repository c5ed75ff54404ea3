// Exact attention forward pass for gfx950 (MI355X, CDNA4).
//
// One workgroup owns one (batch, head, B_r-row query tile) and streams every
// K/V tile of that head through LDS once, keeping per query row a running
// maximum m, a running sum l and an unnormalised output accumulator, all in
// fp32 registers.  Per K/V tile j:
//     S      = Q_i K_j^T                          (MFMA, fp32 accumulate)
//     m_new  = max(m, rowmax S)
//     P      = exp(scale*S - scale*m_new)         (computed as exp2)
//     l      = exp(scale*(m - m_new)) * l + rowsum P
//     O      = exp(scale*(m - m_new)) * O + P V_j (MFMA, P rounded to T)
// and after the last tile O /= l, lse = scale*m + ln l.  This is Algorithm 1
// of FlashAttention-2 ("04 Transformers, Attention, and FlashAttention":
// Q blocks outer and parallel, K/V blocks inner and serial, one division at
// the end, L_i = m_i + log l_i), the row-block recurrence of
// "大语言模型研究14" section 2, and the causal block skipping of
// "FlashAttention 深度解析" (second article, section 2.3).
//
// gfx950 mapping
//  * Each wavefront owns 32 query rows and does every step for them alone, so
//    no row statistic is ever combined across waves.
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_{bf16,f16}: in the 32x32 accumulator layout a lane
//    holds ONE query (its column) and 16 keys, so the row max and row sum are
//    plain in-register max/add chains plus one exchange with lane^32.  (fp16
//    at d = 64 forms the row sum on the matrix core instead, from the rounded
//    P that multiplies V.)
//  * The output is accumulated transposed too, O^T += V^T P^T: the P values a
//    lane holds are exactly the B operand it needs, so P never leaves
//    registers.
//  * 16-bit types (fa_fwd_h_kernel): 8 waves, 256 query rows, 128-key tiles.
//    With fp16 P, m there is a reference that may trail the running maximum
//    by a bounded amount, so O and l are rescaled only when some row's
//    maximum has moved well past it (the reference cancels in O / l and lse).
//    K and V tiles are double-buffered in LDS and filled by LDS-DMA
//    (buffer_load ... lds, no register staging); V^T operands come from
//    row-major V through ds_read_b64_tr_b16.  The two groups of 4 waves run
//    the MFMA work and the softmax of a tile in alternate phases, so each
//    SIMD overlaps one wave's MFMAs with the other wave's VALU work.
//  * fp32 (fa_fwd_f32_kernel): 4 waves, K/V staged through registers into
//    LDS, V written transposed with the 32-key sub-tile's key positions
//    permuted so each lane's 8 keys are one contiguous 16-byte read;
//    v_mfma_f32_32x32x2f32 and P kept in fp32.  On grids too small to fill
//    the chip (d = 64), 8 waves share one 32-row query tile and divide its
//    keys, each keeping its own (m, l, O); the partial states are merged in
//    LDS at the end, as split-K/V partials are.
//  * 16-byte LDS chunks are XOR-swizzled by row to spread banks.
//  * Workgroups are renumbered so that every query tile of a head runs on the
//    same XCD (they share that head's K/V in the XCD's L2); causal tiles are
//    issued heaviest first.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa_detail {
thread_local int g_last_hip = 0;
}  // namespace fa_detail

namespace {

using namespace fa_dev;

// Position of key k (0..31) of a 32-key sub-tile inside a transposed V row.
// The S^T accumulator register r of lane half h holds key 8*(r/4) + 4h + r%4;
// PV step p consumes registers 8p..8p+7.  Swapping bits 2 and 3 of the key
// makes those 8 keys the contiguous positions 16p + 8h .. 16p + 8h + 7.
__device__ inline int vpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

struct Params {
    const char* q;
    const char* k;
    const char* v;
    char* o;
    float* lse;
    int L;
    int BH;
    int Tr;       // query tiles per head
    int remap;    // 1: BH % 8 == 0, keep a head's tiles on one XCD
    float c;      // scale * log2(e)
    float scale;
    // FP8 scores only: per-block scales of Q and K, (BH, nbq) and (BH, nbk)
    // float32, blocks of bq query rows and bk key rows of a head
    const float* qsc;
    const float* ksc;
    int bq, bk, nbq, nbk;
};

template <class T, int D, bool CAUSAL, int NQB, int NW, int NKB>
struct Cfg {
    static constexpr int E = Ty<T>::kBytes;
    static constexpr int QPW = 32 * NQB;          // query rows per wave
    static constexpr int BR = NW * QPW;           // query rows per workgroup
    static constexpr int BC = 32 * NKB;           // keys per K/V tile
    static constexpr int NT = NW * 64;            // threads
    static constexpr int EPC = 16 / E;            // elements per 16-byte chunk
    static constexpr int KCPR = D / EPC;          // chunks per K row (= per V row in HBM)
    static constexpr int VCPR = BC / EPC;         // chunks per transposed-V row
    static constexpr int KSW = (KCPR >= 8 ? 8 : KCPR) - 1;
    static constexpr int VSW = (VCPR >= 8 ? 8 : VCPR) - 1;
    static constexpr int KBYTES = BC * D * E;
    static constexpr int VBYTES = D * BC * E;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KUNITS = BC * KCPR;      // 16-byte pieces of a K tile
    static constexpr int KPT = KUNITS / NT;       // per thread
    static constexpr int VUNITS = (BC / 4) * KCPR;   // (4 keys x 16 bytes) pieces of a V tile
    static constexpr int VPT = (VUNITS + NT - 1) / NT;
    static_assert(KUNITS % NT == 0, "K tile must split evenly over the threads");
    static_assert(D % 32 == 0 && BC % 32 == 0, "tile shapes");
    static_assert(2 * STAGE <= 160 * 1024, "LDS budget");
};

__device__ inline int vswz(int row, int mask) { return (row ^ (row >> 3)) & mask; }

// Which (batch*head, query tile) workgroup blockIdx.x owns.  Dispatch deals
// workgroups round-robin to the 8 XCDs (id % 8); when B*H is a multiple of 8
// the ids are renumbered so that XCD x gets the heads [x*BH/8, (x+1)*BH/8) and
// therefore all of their query tiles, which share K/V through that XCD's L2.
// Non-causal: a head's tiles are consecutive in dispatch order.  Causal: the
// tiles with the most K/V blocks (the last query tiles) are dispatched first.
template <bool CAUSAL>
__device__ inline void work_tile(const Params& p, int& bh, int& qt) {
    const int w = blockIdx.x;
    if (p.remap) {
        const int xcd = w & 7, s = w >> 3, hp = p.BH >> 3;
        if (CAUSAL) {
            qt = p.Tr - 1 - s / hp;
            bh = xcd * hp + s % hp;
        } else {
            bh = xcd * hp + s / p.Tr;
            qt = s % p.Tr;
        }
    } else if (CAUSAL) {
        qt = p.Tr - 1 - w / p.BH;
        bh = w % p.BH;
    } else {
        bh = w / p.Tr;
        qt = w % p.Tr;
    }
}

// SPLIT (small grids): the NW waves share one 32-row query tile and split its
// keys instead of its rows.  Wave w takes the key tiles w, w + NW, ... with
// its own K/V staging in LDS and its own running (m, l, O) over those keys;
// at the end the NW partial states are merged through LDS the way split-K/V
// partials are (each rescaled by exp of its max minus the overall max).
template <class T, int D, bool CAUSAL, int NQB, int NW, int NKB, bool SPLIT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(NQB == 1 ? 2 : 1, NQB == 1 ? 2 : 1)))
void fa_fwd_f32_kernel(Params p) {
    using C = Cfg<T, D, CAUSAL, NQB, NW, NKB>;
    // staging: the whole workgroup fills one tile, or (SPLIT) each wave its own
    using CS = std::conditional_t<SPLIT, Cfg<T, D, CAUSAL, NQB, 1, NKB>, C>;
    using frag = typename Ty<T>::frag;
    constexpr int E = C::E;
    constexpr int BC = C::BC;
    constexpr int BR = SPLIT ? C::QPW : C::BR;
    static_assert(!SPLIT || NQB == 1, "split keys: one query block per wave");
    constexpr int SMEM = SPLIT ? NW * CS::STAGE : 2 * C::STAGE;
    static_assert(SMEM <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    int bh, qt;
    if constexpr (SPLIT) {
        bh = blockIdx.x / p.Tr;
        qt = blockIdx.x % p.Tr;
    } else {
        work_tile<CAUSAL>(p, bh, qt);
    }

    const int L = p.L;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int sid = SPLIT ? lane : tid;               // index among the threads that stage a tile
    const long long head = (long long)bh * L * D;   // element offset of this head
    const char* qh = p.q + head * E;
    const char* kh = p.k + head * E;
    const char* vh = p.v + head * E;

    const int q0 = qt * BR;
    const int qw = SPLIT ? q0 : q0 + wave * C::QPW;   // first query row of this wave
    const int qend = min(q0 + BR, L);
    const int ntiles = CAUSAL ? (qend + BC - 1) / BC : (L + BC - 1) / BC;

    // ---- Q fragments: B operand of S^T = K Q^T, lane = query, 8 d-values ----
    frag qf[NQB][D / 16];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int row = qw + qb * 32 + l32;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            u32x4 raw[E / 2];
#pragma unroll
            for (int x = 0; x < E / 2; ++x) {
                raw[x] = u32x4{0, 0, 0, 0};
                if (row < L) raw[x] = ld16(qh + ((long long)row * D + 16 * s + 8 * hf) * E + 16 * x);
            }
            qf[qb][s] = __builtin_bit_cast(frag, raw);
        }
    }

    // ---- K/V tile prefetch registers ----
    u32x4 kr[CS::KPT];
    u32x4 vr[CS::VPT][4];

    auto fetch = [&](int j) {
        const int kb = j * BC;
#pragma unroll
        for (int x = 0; x < CS::KPT; ++x) {
            const int u = sid + x * CS::NT;
            const int row = u / C::KCPR, c = u % C::KCPR;
            const int key = kb + row;
            kr[x] = u32x4{0, 0, 0, 0};
            if (key < L) kr[x] = ld16(kh + ((long long)key * D) * E + 16 * c);
        }
#pragma unroll
        for (int x = 0; x < CS::VPT; ++x) {
            const int u = sid + x * CS::NT;
            const int a = u / C::KCPR, c = u % C::KCPR;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kb + 4 * a + e;
                vr[x][e] = u32x4{0, 0, 0, 0};
                if (u < CS::VUNITS && key < L) vr[x][e] = ld16(vh + ((long long)key * D) * E + 16 * c);
            }
        }
    };

    // (SPLIT: stage is the wave)
    auto stash = [&](int stage) {
        char* ks = smem + stage * CS::STAGE;
        char* vs = ks + C::KBYTES;
#pragma unroll
        for (int x = 0; x < CS::KPT; ++x) {
            const int u = sid + x * CS::NT;
            const int row = u / C::KCPR, c = u % C::KCPR;
            st16(ks + row * (D * E) + ((c ^ (row & C::KSW)) * 16), kr[x]);
        }
#pragma unroll
        for (int x = 0; x < CS::VPT; ++x) {
            const int u = sid + x * CS::NT;
            if (u >= CS::VUNITS) continue;
            const int a = u / C::KCPR, c = u % C::KCPR;
            const int key4 = 4 * a;                             // 4 consecutive keys
            const int pos = (key4 & ~31) | vpos(key4 & 31);     // their position (contiguous 4)
            const int byte = pos * E;
#pragma unroll
            for (int dd = 0; dd < C::EPC; ++dd) {
                const int drow = c * C::EPC + dd;
                char* dst = vs + drow * (BC * E) + (((byte >> 4) ^ vswz(drow, C::VSW)) << 4) + (byte & 15);
                if constexpr (E == 2) {
                    const int wi = dd >> 1;
                    uint32_t x0 = vr[x][0][wi], x1 = vr[x][1][wi], x2 = vr[x][2][wi], x3 = vr[x][3][wi];
                    u32x2 out;
                    if (dd & 1) {
                        out[0] = (x0 >> 16) | (x1 & 0xffff0000u);
                        out[1] = (x2 >> 16) | (x3 & 0xffff0000u);
                    } else {
                        out[0] = (x0 & 0xffffu) | (x1 << 16);
                        out[1] = (x2 & 0xffffu) | (x3 << 16);
                    }
                    st8(dst, out);
                } else {
                    st16(dst, u32x4{vr[x][0][dd], vr[x][1][dd], vr[x][2][dd], vr[x][3][dd]});
                }
            }
        }
    };

    // ---- running statistics (per lane: one query per qb) and accumulators ----
    float m_raw[NQB], mc[NQB], lsum[NQB];
    f32x16 oacc[NQB][D / 32];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_raw[qb] = -INFINITY;
        mc[qb] = -INFINITY;
        lsum[qb] = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][dt][r] = 0.f;
    }

    // one K/V tile (keys kb ..) from the staged copy at ks
    auto tile = [&](const char* ks, int kb) {
        const char* vs = ks + C::KBYTES;
        // a wave whose rows all precede this tile has nothing to do in it
        const bool active = !CAUSAL || kb <= qw + C::QPW - 1;
        const bool need_mask = (kb + BC > L) || (CAUSAL && kb + BC - 1 > qw);

        if (active) {
            // S^T = K_j Q^T : lane = query, registers = keys
            f32x16 sacc[NQB][NKB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[qb][kt][r] = 0.f;
#pragma unroll
            for (int kt = 0; kt < NKB; ++kt) {
                const int row = kt * 32 + l32;
                const char* krow = ks + row * (D * E);
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    u32x4 raw[E / 2];
#pragma unroll
                    for (int x = 0; x < E / 2; ++x) {
                        const int c = ((16 * s + 8 * hf) * E) / 16 + x;
                        raw[x] = ld16(krow + ((c ^ (row & C::KSW)) * 16));
                    }
                    const frag a = __builtin_bit_cast(frag, raw);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) sacc[qb][kt] = Ty<T>::mma(a, qf[qb][s], sacc[qb][kt]);
                }
            }

            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const int query = qw + qb * 32 + l32;
#pragma unroll
                    for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kb + kt * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
                            if (key >= L || (CAUSAL && key > query)) sacc[qb][kt][r] = -INFINITY;
                        }
                }
            }

            // online softmax update, one query row per lane and qb
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float mx = sacc[qb][0][0];
#pragma unroll
                for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kt][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_raw[qb], mx);
                // reference for the exponent; 0 while the row has seen no key
                const float ref = (m_new == -INFINITY) ? 0.f : m_new * p.c;
                const float alpha = __builtin_amdgcn_exp2f(mc[qb] - ref);
                m_raw[qb] = m_new;
                mc[qb] = ref;
                float ls = 0.f;
#pragma unroll
                for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kt][r], p.c, -ref));
                        sacc[qb][kt][r] = e;
                        ls += e;
                    }
                lsum[qb] = alpha * lsum[qb] + ls;
                if (__ballot(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[qb][dt][r] *= alpha;
                }
            }

            // O^T += V_j^T P^T
#pragma unroll
            for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                for (int ps = 0; ps < 2; ++ps) {
                    frag pb[NQB];
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) {
                        float tmp[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) tmp[e] = sacc[qb][kt][8 * ps + e];
                        pb[qb] = Ty<T>::cvt(tmp);
                    }
                    const int kpos = kt * 32 + 16 * ps + 8 * hf;   // first of this lane's 8 keys
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt) {
                        const int drow = dt * 32 + l32;
                        const char* vrow = vs + drow * (BC * E);
                        u32x4 raw[E / 2];
#pragma unroll
                        for (int x = 0; x < E / 2; ++x) {
                            const int c = (kpos * E) / 16 + x;
                            raw[x] = ld16(vrow + ((c ^ vswz(drow, C::VSW)) * 16));
                        }
                        const frag a = __builtin_bit_cast(frag, raw);
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb) oacc[qb][dt] = Ty<T>::mma(a, pb[qb], oacc[qb][dt]);
                    }
                }
        }

    };

    // SPLIT: merge the waves' partial states.  Wave w leaves its unnormalised
    // O_w (32 rows x D), its exponent reference m_w and its sum l_w; with M the
    // largest m_w of the waves that saw a key (l_w > 0),
    //     O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w,
    //     lse = ln2 * (M + log2 sum_w 2^(m_w - M) l_w).
    auto merge_split = [&]() {
        if constexpr (SPLIT) {
            __syncthreads();                                  // every wave is done with its stage
            float* mo = reinterpret_cast<float*>(smem);       // [NW][32][D]
            float* mm = mo + NW * 32 * D;                     // [NW][32]
            float* ml = mm + NW * 32;                         // [NW][32]
            static_assert((NW * 32 * D + 2 * NW * 32) * 4 <= SMEM, "merge fits the stages");
            const float ltot = lsum[0] + __shfl_xor(lsum[0], 32);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mo[(wave * 32 + l32) * D + dt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)] = oacc[0][dt][r];
            if (hf == 0) {
                mm[wave * 32 + l32] = mc[0];
                ml[wave * 32 + l32] = ltot;
            }
            __syncthreads();
            // thread t: row t / (D/4), columns 4*(t % (D/4)) .. +3
            for (int t = tid; t < 32 * (D / 4); t += NW * 64) {
                const int r = t / (D / 4), c0 = 4 * (t % (D / 4));
                const int query = q0 + r;
                if (query >= L) continue;
                float M = -INFINITY;
                for (int w = 0; w < NW; ++w)
                    if (ml[w * 32 + r] > 0.f) M = fmaxf(M, mm[w * 32 + r]);
                float lt = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
                for (int w = 0; w < NW; ++w) {
                    const float lw = ml[w * 32 + r];
                    if (!(lw > 0.f)) continue;
                    const float f = __builtin_amdgcn_exp2f(mm[w * 32 + r] - M);
                    lt += f * lw;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] += f * mo[(w * 32 + r) * D + c0 + e];
                }
                const float inv = 1.f / lt;
                float o4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = acc[e] * inv;
                st16(p.o + (head + (long long)query * D + c0) * E, __builtin_bit_cast(u32x4, o4));
                if (c0 == 0) p.lse[(long long)bh * L + query] = (M + __builtin_amdgcn_logf(lt)) * kLn2;
            }
        }
    };

    if constexpr (SPLIT) {
        // each wave streams its own tiles: the next one's loads are in flight
        // while the current one is computed (a wave's LDS accesses complete
        // in order, so its stage needs no barrier)
        if (wave < ntiles) fetch(wave);
        for (int j = wave; j < ntiles; j += NW) {
            stash(wave);
            if (j + NW < ntiles) fetch(j + NW);
            tile(smem + wave * CS::STAGE, j * BC);
        }
        merge_split();
        return;
    } else {
        fetch(0);
        stash(0);
        __syncthreads();
        for (int j = 0; j < ntiles; ++j) {
            if (j + 1 < ntiles) fetch(j + 1);
            tile(smem + (j & 1) * C::STAGE, j * BC);
            if (j + 1 < ntiles) stash((j + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogue: one division by l, logsumexp, stores ----
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const float ltot = lsum[qb] + __shfl_xor(lsum[qb], 32);
        const float inv = 1.f / ltot;
        const int query = qw + qb * 32 + l32;
        if (query < L) {
            char* orow = p.o + (head + (long long)query * D) * E;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = dt * 32 + g * 8 + hf * 4;
                    if constexpr (E == 2) {
                        T o4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[qb][dt][4 * g + e] * inv);
                        st8(orow + col * E, __builtin_bit_cast(u32x2, o4));
                    } else {
                        float o4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) o4[e] = oacc[qb][dt][4 * g + e] * inv;
                        st16(orow + col * E, __builtin_bit_cast(u32x4, o4));
                    }
                }
            if (hf == 0) p.lse[(long long)bh * L + query] = (mc[qb] + __builtin_amdgcn_logf(ltot)) * kLn2;
        }
    }
}

// ===========================================================================
// 16-bit inputs (bf16, fp16)
//
// Same per-wave arithmetic as above, with the K/V staging reworked for gfx950:
//  * K and V tiles go HBM -> LDS with buffer_load_dwordx4 ... lds (no register
//    staging, no ds_write).  The buffer descriptor spans exactly one head, so
//    rows past L read as zeros.
//  * V stays row-major in LDS; the A operand of O^T += V^T P^T is read with
//    ds_read_b64_tr_b16, which hands each lane 4 keys of one d column.  In a
//    16-lane group, lane i receives element i%4 of the 8 bytes addressed by
//    lane 4e+i/4 as its element e; so lane 16g+4e+q addresses key row e of its
//    4-key group, d columns 4q..4q+3 of its 16-column band.
//  * 16-byte chunks are XOR-swizzled per row (K: 16 consecutive rows hit 16
//    different bank slots with one chunk index; V: 4 consecutive rows spread a
//    64-byte column band over all slots).  The DMA writes 1 KB per wave
//    instruction contiguously, so each lane fetches the global chunk that
//    belongs at its LDS slot.
//  * Every per-lane LDS offset is computed once; the loop adds only
//    immediates.
// ===========================================================================


#ifndef FA_H_NKB128
#define FA_H_NKB128 4
#endif
#ifndef FA_H_NKB64
#define FA_H_NKB64 4
#endif

// Tile shape of the 16-bit-V kernel: 8 waves x 32 query rows, 32*NKB-key
// tiles.  FP8: Q and K are one-byte E4M3 codes, V stays 16-bit.
template <int D, bool FP8 = false>
struct HCfg {
    static constexpr int NW = 8, QPW = 32, BR = NW * QPW, NKB = (D == 128 ? FA_H_NKB128 : FA_H_NKB64), BC = 32 * NKB;
    static constexpr int P = D * 2;                 // V row pitch in LDS (bytes)
    static constexpr int PK = FP8 ? D : D * 2;      // Q and K row pitch (bytes)
    static constexpr int TILE = BC * P;             // one V tile (bytes)
    static constexpr int TILEK = BC * PK;           // one K tile (bytes)
    static constexpr int LPW = TILE / 1024 / NW;    // 1 KB DMA instructions per wave per V tile
    static constexpr int LPWK = TILEK / 1024 / NW;  // ... per K tile
    static_assert(LPWK >= 1 && LPWK * NW * 1024 == TILEK, "tile must split into 1 KB pieces per wave");
    static_assert(LPW >= 1 && LPW * NW * 1024 == TILE, "tile must split into 1 KB pieces per wave");
    // LDS: K stage 0, K stage 1, V stage 0, V stage 1; FP8 adds four 256-byte
    // slots for the K tiles' block scales
    static constexpr int SCOFF = 2 * TILEK + 2 * TILE;
    static constexpr int BYTES = SCOFF + (FP8 ? 4 * 256 : 0);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Row layout of an FP8 K tile (rows of D bytes, 16-byte chunks XOR-swizzled):
// the 16 rows one 16-lane pass of ds_read_b128 reads start in 256/D distinct
// bank positions, and the swizzle gives rows sharing a position distinct
// chunks, so a pass touches all 64 banks once.
template <int D>
struct K8Layout {
    static constexpr int CPR = D / 16, RPB = 256 / D;
    __device__ static inline int fk(int r) { return (r / RPB) & (CPR - 1); }
};

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row sums of P on the matrix core.  v_mfma_f32_16x16x32_f16 reads a lane's P
// fragment (the 32x32x16 B operand: query l % 32, 8 keys) as column l % 16 of
// k-group l / 16, so query q's fragments sit in k-groups 0 and 2 of column q
// (q < 16) or in k-groups 1 and 3 of column q - 16.  This A operand has ones
// in row 0 over k-groups 0 and 2 (lanes 0, 32) and in row 4 over k-groups 1
// and 3 (lanes 20, 52), zeros elsewhere; the product then holds query q's sum
// in row 0 or 4 of column q % 16, which the 16x16 result layout puts in
// register 0 of lane q.  Lanes 32-63 hold zeros.
__device__ inline f16x8 row_sum_selector(int lane) {
    const bool one = lane == 0 || lane == 32 || lane == 20 || lane == 52;
    f16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = one ? (_Float16)1.f : (_Float16)0.f;
    return a;
}

// S^T += K Q^T over 64 d-values with E4M3 codes: the K row chunks (a0, a1)
// and Q row chunks (b0, b1) hold 32 consecutive d-values of the lane's
// half.  gfx950's f8f6f4 MFMA with format 0 (E4M3) for both operands and
// no block scaling.
__device__ inline f32x16 mma_e4m3(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
    const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// LDS-DMA of one dword per lane: lane l's 4 bytes land at lds_base + 4l
// (the same explicit-wait contract as dma16).
__device__ inline void dma4(i32x4 rsrc, int voff, unsigned lds_base) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(voff), "s"(rsrc)
        : "memory");
}

template <class F>
__device__ inline f32x16 mma_e4m3(F a0, F a1, F b0, F b1, f32x16 c) {
    return mma_e4m3(__builtin_bit_cast(u32x4, a0), __builtin_bit_cast(u32x4, a1), __builtin_bit_cast(u32x4, b0),
                    __builtin_bit_cast(u32x4, b1), c);
}

// Issue order of the MFMA slices of one phase: the NPV slices of P V (whose
// operands come from transposing LDS reads, the slower kind) are spread
// evenly among the NS score slices so LDS demand stays level.
template <int NPV, int NS>
struct SliceOrder {
    int v[NPV + NS > 0 ? NPV + NS : 1];
    constexpr SliceOrder() : v{} {
        int p = 0, s = 0;
        for (int i = 0; i < NPV + NS; ++i) {
            if (s >= NS || (p < NPV && p * NS <= s * NPV)) v[i] = p++;
            else v[i] = NPV + s++;
        }
    }
};

// Whether any of the lane's fp16 P values (all >= 0, or +inf where a value
// overflowed) exceeds lim: a packed maximum over the P registers,
// v_pk_maximum3_f16 taking two registers (four values) per instruction.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <class F, int N>
__device__ inline bool p16_above(const F (&pf)[N][2], _Float16 lim) {
    f16x2 m = {(_Float16)0.f, (_Float16)0.f};
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f16x8 v = __builtin_bit_cast(f16x8, pf[i][h]);
            m = __builtin_elementwise_maximum(m, __builtin_shufflevector(v, v, 0, 1));
            m = __builtin_elementwise_maximum(m, __builtin_shufflevector(v, v, 2, 3));
            m = __builtin_elementwise_maximum(m, __builtin_shufflevector(v, v, 4, 5));
            m = __builtin_elementwise_maximum(m, __builtin_shufflevector(v, v, 6, 7));
        }
    return __builtin_elementwise_maximum(m[0], m[1]) > lim;
}

// How far (in base-2 units of scaled scores) the reference a row's P is taken
// against may trail the row's running maximum.  The reference cancels in O / l
// and in lse = ref + log l, so in exact arithmetic any value gives the same
// result, and a trail of at most 8 keeps P <= 256, far inside the 16-bit
// range, while sparing the rescale of O in most tiles once the maxima have
// settled.  In rounded arithmetic it costs the exactness of the dominant
// weight: with the reference at the maximum that weight is exactly 1, with a
// trailing one it is 2^delta rounded to the P type, a relative error of up to
// half an ulp of that type which shows in rows one key dominates.  fp16 P
// (11 significant bits) keeps that near the rounding of O itself; bf16 P (8)
// would not, so bf16 keeps the reference at the maximum.
template <class T>
constexpr float ref_lag() { return std::is_same<T, _Float16>::value ? 8.f : 0.f; }

// Ping-pong schedule.  The 8 waves form two groups of 4 (waves 0-3 and 4-7);
// each SIMD runs one wave of each group.  Per K/V tile j a wave has
//     M(j): O^T += V_{j-1}^T P_{j-1}^T  and  S_j = K_j Q^T        (MFMA)
//     X(j): row max, rescale, P_j = exp2(scale*S_j - ref), l     (VALU)
// (fp16 at d = 64 adds P_{j-1}'s row sums to l in M(j), on the matrix core)
// and the groups run them in alternate phases fenced by workgroup barriers:
//     phase   0    1    2    3   ...  2T   2T+1
//     group 0 M(0) X(0) M(1) X(1) ... M(T)  -
//     group 1  -   M(0) X(0) M(1) ... X(T-1) M(T)
// so while one wave of a SIMD feeds the matrix core the other keeps the VALU
// busy with the softmax.  M(T) only finishes the last PV.  K_j and V_{j-1}
// are read in phases 2j and 2j+1; the DMA for K_{j+1} and V_j goes into the
// other stages during phase 2j and is complete by the end of phase 2j+1.
template <class T, int D, bool CAUSAL, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512))) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_h_kernel(Params p) {
    using Cf = HCfg<D, FP8>;
    constexpr int QPW = Cf::QPW, BR = Cf::BR, NKB = Cf::NKB, BC = Cf::BC;
    constexpr int P = Cf::P, TILE = Cf::TILE, LPW = Cf::LPW;
    constexpr int PK = Cf::PK, TILEK = Cf::TILEK, LPWK = Cf::LPWK;
    using Lay = HLayout<D>;
    using frag = typename Ty<T>::frag;
    // 16-byte chunks of one Q or K row a lane holds for the score MFMAs:
    // 16-bit, one per 16-wide d step; FP8, two per 64-wide d step
    constexpr int NQC = FP8 ? D / 32 : D / 16;

    __shared__ __attribute__((aligned(1024))) char smem[Cf::BYTES];

    int bh, qt;
    work_tile<CAUSAL>(p, bh, qt);

    const int L = p.L;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int group = wave >> 2;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const long long head = (long long)bh * L * D;
    const char* qh = p.q + head * (PK / D);
    const char* kh = p.k + head * (PK / D);
    const char* vh = p.v + head * 2;
    const i32x4 krs = buffer_rsrc(kh, L * PK);

    const int q0 = qt * BR;
    const int qw = q0 + wave * QPW;                 // this wave's first query row
    const int qend = min(q0 + BR, L);
    const int ntiles = CAUSAL ? (qend + BC - 1) / BC : (L + BC - 1) / BC;   // K/V tiles of the workgroup
    // K/V tiles this wave computes (0 for a wave entirely past L)
    const int ntw = qw >= L ? 0 : (CAUSAL ? (min(qw + QPW, L) + BC - 1) / BC : ntiles);

    // Q fragments (B operand of S^T = K Q^T).  Chunk s of the lane: 16-bit,
    // elements 16s + 8hf .. +7; FP8, bytes 64(s/2) + 32hf + 16(s%2) .. +15.
    frag qf[NQC];
    {
        const int row = qw + l32;
#pragma unroll
        for (int s = 0; s < NQC; ++s) {
            u32x4 raw = u32x4{0, 0, 0, 0};
            if constexpr (FP8) {
                if (row < L) raw = ld16(qh + (long long)row * PK + 64 * (s >> 1) + 32 * hf + 16 * (s & 1));
            } else {
                if (row < L) raw = ld16(qh + ((long long)row * D + 16 * s + 8 * hf) * 2);
            }
            qf[s] = __builtin_bit_cast(frag, raw);
        }
        // take the Q loads' wait here, once, instead of inside the K/V loop
#pragma unroll
        for (int s = 0; s < NQC; ++s) asm volatile("" : "+v"(qf[s]));
    }
    // FP8: this lane's query-block scale times scale*log2(e)
    float cq = p.c;
    if constexpr (FP8) {
        cq = p.c * p.qsc[(long long)bh * p.nbq + min(qw + l32, L - 1) / p.bq];
        asm volatile("" : "+v"(cq));
    }

    // DMA mapping: byte o = 1024*n + 16*lane of a tile holds row o/P, slot
    // (o%P)/16, i.e. global chunk slot ^ f(row) of that row.  One wave of the
    // issuing group covers the 1 KB pieces n = (wave & 3)*LPW + x of wave
    // (wave & 3) and the same pieces of wave (wave & 3) + 4, 4096*LPW bytes on.
    // Over x the K offsets differ by 1024*x in the row bits and 4*x in the
    // swizzled chunk, bits disjoint from the rest (the K swizzle of row
    // 4x + g is 4x | g at d = 128 and (4x | g) & 7 at d = 64), so piece x is
    // kd0 ^ (x * 0x440); the V swizzle repeats every 4 rows, so its piece x
    // is vd0 + 1024*x.
    const int wq = wave & 3;
    int kd0, vd0;
    {
        const int o = 1024 * (wq * LPW) + 16 * lane;
        const int r = o / P, slot = (o % P) >> 4;
        kd0 = r * P + ((slot ^ Lay::fk(r)) << 4);
        vd0 = r * P + ((slot ^ Lay::fv(r)) << 4);
        if constexpr (FP8) {        // K rows of D bytes, same 4-rows-per-piece-step argument
            const int ok = 1024 * (wq * LPWK) + 16 * lane;
            const int rk = ok / PK, slotk = (ok % PK) >> 4;
            kd0 = rk * PK + ((slotk ^ K8Layout<D>::fk(rk)) << 4);
        }
    }
    auto kdma_off = [&](int x, int hi) { return (kd0 ^ (x * 0x440)) + hi * 4096 * LPWK; };
    auto vdma_off = [&](int x, int hi) { return vd0 + 1024 * x + hi * 4096 * LPW; };
    const unsigned lds0 = (unsigned)(unsigned long long)(lds_char*)smem;
    // FP8: the block scales of K tile t's NKB sub-tiles go to LDS slot t & 3
    // (lane kt fetches sub-tile kt's; the slot is read in X(t), so it must
    // outlive the stage of K_t by one phase: four slots)
    i32x4 ksrs = i32x4{0, 0, 0, 0};
    if constexpr (FP8) ksrs = buffer_rsrc(p.ksc + (long long)bh * p.nbk, p.nbk * 4);
    auto issue_ksc = [&](int t) {
        if constexpr (FP8) {
            const int kt = lane < NKB ? lane : 0;
            const int idx = min(t * BC + 32 * kt, L - 1) / p.bk;
            dma4(ksrs, idx * 4, __builtin_amdgcn_readfirstlane(lds0 + Cf::SCOFF + (t & 3) * 256));
        }
    };
    auto issue_k2 = [&](int j) {
        issue_ksc(j);
        const unsigned dst = lds0 + (j & 1) * TILEK + 1024 * wq * LPWK;
#pragma unroll
        for (int x = 0; x < LPWK; ++x) {
            dma16(krs, kdma_off(x, 0) + j * TILEK, __builtin_amdgcn_readfirstlane(dst + 1024 * x));
            dma16(krs, kdma_off(x, 1) + j * TILEK, __builtin_amdgcn_readfirstlane(dst + 4096 * LPWK + 1024 * x));
        }
    };
    // per-lane LDS read offsets
    // K chunk s of the lane (as for qf): 16-bit chunk 2s + hf of row l32;
    // FP8 chunk 4(s/2) + 2hf + s%2
    int koff[NQC];
#pragma unroll
    for (int s = 0; s < NQC; ++s) {
        if constexpr (FP8) koff[s] = l32 * PK + (((4 * (s >> 1) + 2 * hf + (s & 1)) ^ K8Layout<D>::fk(l32)) << 4);
        else koff[s] = l32 * P + (((2 * s + hf) ^ Lay::fk(l32)) << 4);
    }
    int voffv[D / 32];
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
        const int rrel = 4 * (g >> 1) + e;            // key row within an 8-key group
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int c = 4 * dt + 2 * (g & 1) + (q >> 1);
            voffv[dt] = 2 * TILEK + rrel * P + ((c ^ Lay::fv(rrel)) << 4) + 8 * (q & 1);   // V stages start at 2*TILEK
        }
    }

    float mc = -INFINITY, lsum = 0.f;
    // fp16 at d = 64, where the softmax's VALU work bounds the kernel and the
    // matrix core has room: l is the row sum of the rounded P (the weights
    // P V uses), accumulated on the matrix core beside P V in lacc, instead
    // of 64 VALU adds per lane and tile into lsum
    constexpr bool LMMA = std::is_same<T, _Float16>::value && D == 64;
    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
    const f16x8 lsel = row_sum_selector(lane);
    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    f32x16 sacc[NKB];
    frag pf[NKB][2];            // P of the last softmax phase, as MFMA B operands

    // Group 0 issues every K/V DMA, from its MFMA phases: in M(t) (phase 2t)
    // the 1 KB pieces of K_{t+1} and V_t go out one or two after each MFMA
    // slice, where the wave otherwise waits on the matrix core, and group 0
    // waits for them at the end of its X(t) (phase 2t+1); the barrier there
    // publishes the stages, which are first read in phase 2t+2.
    const bool feeder = group == 0;
    constexpr int NPIECE = 2 * LPWK + 2 * LPW + (FP8 ? 1 : 0);   // DMA instructions per wave for K_{t+1}, V_t
    auto dma_piece = [&](int t, int n) {          // n-th instruction of K_{t+1}, V_t
        const int hi = n & 1;
        // the descriptors move to the tile, so the per-lane offsets are loop-invariant
        if (n < 2 * LPWK) {
            const int x = n >> 1;
            if (t + 1 < ntiles) {
                const unsigned dst = lds0 + ((t + 1) & 1) * TILEK + 1024 * (wq * LPWK + x) + hi * 4096 * LPWK;
                dma16(buffer_rsrc_at(kh, L * PK, (t + 1) * TILEK), kdma_off(x, hi),
                      __builtin_amdgcn_readfirstlane(dst));
            }
        } else if (FP8 && n == NPIECE - 1) {
            if (t + 1 < ntiles) issue_ksc(t + 1);
        } else {
            const int x = (n - 2 * LPWK) >> 1;
            const unsigned dst = lds0 + 2 * TILEK + (t & 1) * TILE + 1024 * (wq * LPW + x) + hi * 4096 * LPW;
            dma16(buffer_rsrc_at(vh, L * P, t * TILE), vdma_off(x, hi), __builtin_amdgcn_readfirstlane(dst));
        }
    };
    auto dma_tile = [&](int t) {                  // all of K_{t+1}, V_t at once (phases without MFMAs)
#pragma unroll
        for (int n = 0; n < NPIECE; ++n) dma_piece(t, n);
    };
    // after MFMA slice pos of nsl in M(t): its share of the pieces
    auto mfeed = [&](int t, int pos, int nsl) {
        if (feeder && t < ntiles) {
            const int n0 = (pos * NPIECE + nsl - 1) / nsl, n1 = ((pos + 1) * NPIECE + nsl - 1) / nsl;
#pragma unroll
            for (int n = n0; n < n1; ++n) dma_piece(t, n);
        }
    };

    // M(j): PV of tile j-1, scores of tile j.  The MFMAs run in slices of
    // up to 4 (PV: one 8-key slice of P against the D/32 tiles of V^T;
    // scores: 4 d-steps of one 32-key sub-tile), PV slices spread among the
    // score slices.  The operands of slice i+1 are read from LDS while
    // slice i runs: after each MFMA of slice i goes its share of those reads,
    // so that reads neither queue behind a burst nor land just before use.
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using PR = std::integral_constant<int, -1>;
    // par_tag: K/V stage parity of tile j when known at compile time (0/1),
    // else -1; a known parity folds the stage offsets into the LDS reads
    auto mma_run = [&](auto pv_tag, auto s_tag, int j, auto par_tag) {
        constexpr bool PV = decltype(pv_tag)::value;
        constexpr bool SC = decltype(s_tag)::value;
        constexpr int PAR = decltype(par_tag)::value;
        constexpr int GPT = FP8 ? 1 : D / 64;             // score slices per 32-key sub-tile
        constexpr int NPV = PV ? 2 * NKB : 0;
        constexpr int NSL = NPV + (SC ? NKB * GPT : 0);
        constexpr SliceOrder<NPV, NSL - NPV> ord{};
        // the MFMA wave of a SIMD takes issue priority; the softmax wave
        // sharing the SIMD fills the gaps
        __builtin_amdgcn_s_setprio(3);
        const int kst = PAR >= 0 ? PAR : (j & 1);
        const lds_char* vs = (const lds_char*)smem + (1 - kst) * TILE;    // voffv holds the 2*TILEK
        const char* ks = smem + kst * TILEK;
        frag buf[2][4];
        auto load = [&](int pos) {
            const int i = ord.v[pos];
            if (i < NPV) {
                const int rowb = ((i >> 1) * 32 + 16 * (i & 1)) * P;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vs + rowb + voffv[dt]));
                    const v4i16 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vs + rowb + 8 * P + voffv[dt]));
                    buf[pos & 1][dt] = __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            } else if constexpr (FP8) {
                const int kt = i - NPV;
#pragma unroll
                for (int x = 0; x < NQC; ++x)
                    buf[pos & 1][x] = __builtin_bit_cast(frag, ld16(ks + kt * 32 * PK + koff[x]));
            } else {
                const int g = i - NPV, kt = g / GPT, s0 = 4 * (g % GPT);
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    buf[pos & 1][x] = __builtin_bit_cast(frag, ld16(ks + kt * 32 * P + koff[s0 + x]));
            }
        };
        auto exec = [&](int pos) {
            const int i = ord.v[pos];
            if (i < NPV) {
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = Ty<T>::mma(buf[pos & 1][dt], pf[i >> 1][i & 1], oacc[dt]);
                if constexpr (LMMA)
                    lacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lsel, __builtin_bit_cast(f16x8, pf[i >> 1][i & 1]),
                                                                 lacc, 0, 0, 0);
            } else if constexpr (FP8) {
                const int kt = i - NPV;
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
                for (int m = 0; m < D / 64; ++m)
                    sacc[kt] = mma_e4m3(buf[pos & 1][2 * m], buf[pos & 1][2 * m + 1], qf[2 * m], qf[2 * m + 1], sacc[kt]);
            } else {
                const int g = i - NPV, kt = g / GPT, s0 = 4 * (g % GPT);
                if (s0 == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) sacc[kt] = Ty<T>::mma(buf[pos & 1][x], qf[s0 + x], sacc[kt]);
            }
        };
        load(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
            const bool more = i + 1 < NSL;
            if (more) load(i + 1);
            exec(i);
            mfeed(j, i, NSL);
            if (more && !FP8) {
                const int rd = ord.v[i + 1] < NPV ? 2 : 1;    // LDS reads per MFMA
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                    if (rd == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // then LDS reads
                    else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                if (LMMA && ord.v[i] < NPV) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the row sums
            } else if (more) {
                // FP8 score slices hold D/64 (longer) MFMAs and D/32 reads;
                // PV slices D/32 MFMAs with two reads each
                const int nm = ord.v[i] < NPV ? D / 32 : D / 64;
                const int rd = (ord.v[i + 1] < NPV ? D / 16 : D / 32) / nm;
#pragma unroll
                for (int x = 0; x < nm; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (rd == 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                    else if (rd == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // X(j): online-softmax update for tile j (MASK: the tile reaches past L
    // or past this wave's first query); leaves P_j in pf
    auto softmax_run = [&](auto mask_tag, int j) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int kb = j * BC;
        __builtin_amdgcn_s_setprio(0);
        if constexpr (MASK) {
            // register r of sub-tile kt holds key kb + 4*hf + c with the
            // constant c = 32*kt + 8*(r/4) + r%4; the key is masked when it is
            // past the query (causal) or past L-1, i.e. when c > lim
            const int last = CAUSAL ? min(qw + l32, L - 1) : L - 1;
            const int lim = last - kb - 4 * hf;
#pragma unroll
            for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kt + 8 * (r >> 2) + (r & 3) > lim) sacc[kt][r] = -INFINITY;
        }
        // score factor per 32-key sub-tile: scale*log2(e), times the query
        // and key block scales for FP8 (one key block per sub-tile)
        float ck[NKB];
#pragma unroll
        for (int kt = 0; kt < NKB; ++kt) ck[kt] = p.c;
        if constexpr (FP8) {
            const float* ks = reinterpret_cast<const float*>(smem + Cf::SCOFF + (j & 3) * 256);
#pragma unroll
            for (int kt = 0; kt < NKB; ++kt) ck[kt] = cq * ks[kt];
        }
        // the exact row maximum of the tile's scores, in scaled log2 units
        auto row_max = [&]() -> float {
            float mx;
            if constexpr (FP8) {
                mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < NKB; ++kt) {
                    float m = sacc[kt][0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) m = fmaxf(m, sacc[kt][r]);
                    mx = fmaxf(mx, m * ck[kt]);
                }
            } else {
                mx = sacc[0][0];
#pragma unroll
                for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
            }
            return FP8 ? pair_max(mx) : pair_max(mx) * p.c;
        };
        constexpr float lag = ref_lag<T>();
        auto rescale = [&](float alpha) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        };
        // fp16 P at d = 64 (where the softmax bounds the kernel and the
        // registers allow the scores to stay live while P is formed): P is
        // formed against the trailing reference first, and the row maxima
        // only when some P of the wave exceeds 2^lag or a row has no
        // reference yet.  The test is a packed fp16 maximum over the P
        // registers, half the instructions of the fp32 maximum over the
        // scores.  Elsewhere the row maxima come first.
        constexpr bool PFIRST = lag > 0.f && D == 64;
        if constexpr (PFIRST) {
            auto form_p = [&](float& ts) {
                const float ref = (mc == -INFINITY) ? 0.f : mc;
#pragma unroll
                for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
                    for (int ps = 0; ps < 2; ++ps) {
                        float pe[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            pe[e] = __builtin_amdgcn_exp2f(
                                __builtin_fmaf(sacc[kt][8 * ps + e], FP8 ? ck[kt] : p.c, -ref));
                            if constexpr (!LMMA) ts += pe[e];
                        }
                        pf[kt][ps] = Ty<T>::cvt(pe);
                    }
            };
            float ts = 0.f;
            form_p(ts);
            if (__ballot(p16_above(pf, (_Float16)__builtin_exp2f(lag)) || mc == -INFINITY)) {
                const float cand = row_max();
                const bool bump = cand > mc;
                const float alpha = bump ? __builtin_amdgcn_exp2f(mc - cand) : 1.f;
                mc = bump ? cand : mc;
                lsum *= alpha;
                rescale(alpha);
                if constexpr (LMMA) lacc[0] *= alpha;
                ts = 0.f;
                form_p(ts);
            }
            if constexpr (!LMMA) lsum += ts;
            return;
        }
        // reference mc in scaled log2 units (-inf while no key is seen).  It
        // trails the running max by at most lag: O and l are rescaled, and
        // every row's mc brought up to its max, only in tiles where some row
        // of the wave passed its mc by more than that
        const float cand = row_max();
        if constexpr (lag > 0.f) {
            if (__ballot(cand > mc + lag)) {
                const bool bump = cand > mc;
                const float alpha = bump ? __builtin_amdgcn_exp2f(mc - cand) : 1.f;
                mc = bump ? cand : mc;
                lsum *= alpha;
                rescale(alpha);
                if constexpr (LMMA) lacc[0] *= alpha;
            }
        } else {
            const bool bump = cand > mc;
            const float alpha = bump ? __builtin_amdgcn_exp2f(mc - cand) : 1.f;
            mc = bump ? cand : mc;
            lsum *= alpha;
            if (__ballot(bump)) {
                rescale(alpha);
                if constexpr (LMMA) lacc[0] *= alpha;
            }
        }
        const float ref = (mc == -INFINITY) ? 0.f : mc;
#pragma unroll
        for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                float pe[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * ps + e], FP8 ? ck[kt] : p.c, -ref));
                    if constexpr (!LMMA) lsum += pe[e];
                }
                pf[kt][ps] = Ty<T>::cvt(pe);
            }
    };

    // The softmax phase's results are consumed only in the next MFMA phase, so
    // the compiler would sink the exp / convert / sum work past the barrier
    // into it.  An empty asm that "modifies" them pins that work here.
    auto pin_x = [&]() {
#pragma unroll
        for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) asm volatile("" : "+v"(pf[kt][ps]));
        asm volatile("" : "+v"(lsum), "+v"(mc));
    };
    // phase boundaries: the scheduling barriers keep the compiler from
    // moving register-only work (row max, MFMAs) across the workgroup barrier,
    // which would undo the phase split
    auto end_m = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto end_x = [&]() {
        pin_x();
        __builtin_amdgcn_sched_barrier(0);
        if (feeder) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    // first tile whose keys can reach past L or past this wave's first query
    const int jmask = CAUSAL ? min(qw / BC, (L - 1) / BC) : (L - 1) / BC;

    if (feeder) issue_k2(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (group == 1) __syncthreads();              // group 1 starts one phase later
    int j = 0;
    if (ntw > 0) {
        mma_run(no{}, yes{}, 0, P0{});
        end_m();
        if (jmask == 0) softmax_run(yes{}, 0);
        else softmax_run(no{}, 0);
        end_x();
        // steady state, no masking; two tiles per trip so that the stage
        // parity (odd j first) is a constant in each half
        const int jsteady = min(jmask, ntw);
        for (j = 1; j + 1 < jsteady; j += 2) {
            mma_run(yes{}, yes{}, j, P1{});
            end_m();
            softmax_run(no{}, j);
            end_x();
            mma_run(yes{}, yes{}, j + 1, P0{});
            end_m();
            softmax_run(no{}, j + 1);
            end_x();
        }
        if (j < jsteady) {
            mma_run(yes{}, yes{}, j, P1{});
            end_m();
            softmax_run(no{}, j);
            end_x();
            ++j;
        }
        for (j = max(j, 1); j < ntw; ++j) {      // tiles that need the mask
            mma_run(yes{}, yes{}, j, PR{});
            end_m();
            softmax_run(yes{}, j);
            end_x();
        }
        mma_run(yes{}, no{}, j, PR{});                  // j == ntw: last PV
        if (j < ntiles || group == 0) end_m();
        if (j < ntiles) end_x();
        ++j;
    }
    for (; j <= ntiles; ++j) {                    // phases of tiles this wave does not need
        if (feeder && j < ntiles) dma_tile(j);
        if (j < ntiles || group == 0) end_m();
        if (j < ntiles) end_x();
    }
    // The last phase (group 1's final P V) needs no barrier after it: group 0
    // goes on to its epilogue, which touches no LDS, while group 1 finishes;
    // each wave has now passed the same number of barriers.

    // epilogue: one division by l, logsumexp, stores
    const float ltot = pair_sum(LMMA ? lacc[0] : lsum);
    const float inv = 1.f / ltot;
    const int query = qw + l32;
    if (query < L) {
        char* orow = p.o + (head + (long long)query * D) * 2;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                T a4[4], b4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a4[e] = (T)(oacc[dt][8 * gp + e] * inv);
                    b4[e] = (T)(oacc[dt][8 * gp + 4 + e] * inv);
                }
                store_chunk_pair<T>(orow, 4 * dt + 2 * gp, hf, a4, b4);
            }
        if (hf == 0) p.lse[(long long)bh * L + query] = (mc + __builtin_amdgcn_logf(ltot)) * kLn2;
    }
}

// ---- host side ----


struct Tiling {
    int br, bc;
};

// Tile shapes: 16-bit types (and FP8 scores) use fa_fwd_h_kernel (8 waves x
// 32 query rows, 128-key tiles); fp32 uses fa_fwd_f32_kernel (4 waves x 32
// query rows; 64-key tiles at d = 64, 32-key tiles at d = 128 for the LDS
// budget).  At d = 64, an fp32 grid of fewer than kF32SplitBelow such
// workgroups leaves most of the chip idle while each wave runs all of its
// keys through its SIMD's fp32 matrix core in series; there the kernel runs
// in its SPLIT form instead: 32-row workgroups of 8 waves that divide the
// keys (32-key tiles) and merge their partial states.
template <class T, int D>
struct F32Choice {
    static constexpr int NQB = 1, NW = 4, NKB = (D == 64 ? 2 : 1);
    using C = Cfg<float, D, false, NQB, NW, NKB>;
};
constexpr int kF32SplitWaves = 8;
constexpr long long kF32SplitBelow = 128;

template <class T, int D>
bool f32_split(int BH, int L) {
    return sizeof(T) == 4 && D == 64 &&
           (long long)BH * ((L + F32Choice<T, D>::C::BR - 1) / F32Choice<T, D>::C::BR) < kF32SplitBelow;
}

template <class T, int D, bool CAUSAL>
Tiling tiling_of(int BH, int L) {
    if constexpr (sizeof(T) == 2) return Tiling{HCfg<D>::BR, HCfg<D>::BC};
    if (f32_split<T, D>(BH, L)) return Tiling{32, 32};
    using C = typename F32Choice<T, D>::C;
    return Tiling{C::BR, C::BC};
}

inline Params make_params(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int L,
                          float scale, int br) {
    Params p;
    p.q = static_cast<const char*>(q);
    p.k = static_cast<const char*>(k);
    p.v = static_cast<const char*>(v);
    p.o = static_cast<char*>(o);
    p.lse = lse;
    p.L = L;
    p.BH = BH;
    p.Tr = (L + br - 1) / br;
    p.remap = (BH % 8 == 0) ? 1 : 0;
    p.c = scale * kLog2e;
    p.scale = scale;
    p.qsc = nullptr;
    p.ksc = nullptr;
    p.bq = p.bk = p.nbq = p.nbk = 1;
    return p;
}

template <class T, int D, bool CAUSAL>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int L, float scale,
           hipStream_t stream) {
    const Tiling t = tiling_of<T, D, CAUSAL>(BH, L);
    const Params p = make_params(q, k, v, o, lse, BH, L, scale, t.br);
    const long long grid = (long long)BH * p.Tr;
    if constexpr (sizeof(T) == 2) {
        return fa_detail::launch_kernel(fa_fwd_h_kernel<T, D, CAUSAL, false>, dim3((unsigned)grid),
                                        dim3(HCfg<D>::NW * 64), stream, p);
    } else if (f32_split<T, D>(BH, L)) {
        if constexpr (D == 64)
            return fa_detail::launch_kernel(fa_fwd_f32_kernel<float, D, CAUSAL, 1, kF32SplitWaves, 1, true>,
                                            dim3((unsigned)grid), dim3(kF32SplitWaves * 64), stream, p);
        return FA_ERR_UNSUPPORTED;
    } else {
        using Ch = F32Choice<T, D>;
        return fa_detail::launch_kernel(fa_fwd_f32_kernel<float, D, CAUSAL, Ch::NQB, Ch::NW, Ch::NKB>,
                                        dim3((unsigned)grid), dim3(Ch::C::NT), stream, p);
    }
}

template <class T>
Tiling tiling_for(int BH, int L, int d, int causal) {
    if (d == 64) return causal ? tiling_of<T, 64, true>(BH, L) : tiling_of<T, 64, false>(BH, L);
    return causal ? tiling_of<T, 128, true>(BH, L) : tiling_of<T, 128, false>(BH, L);
}

// BH = B*H: the fp32 shape depends on the grid size (callers have checked
// that B*H fits an int)
Tiling tiling_dispatch(int BH, int L, int d, int causal, int dtype) {
    if (dtype == FA_F32) return tiling_for<float>(BH, L, d, causal);
    if (dtype == FA_F16) return tiling_for<_Float16>(BH, L, d, causal);
    return tiling_for<__bf16>(BH, L, d, causal);
}

int check_args(int B, int H, int L, int d, int causal, int dtype) {
    if (B <= 0 || H <= 0 || L <= 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const long long n = (long long)B * H * L;
    if (n >= (1LL << 62) / d) return FA_ERR_INVALID_ARG;
    // one head's tensor must stay below 2 GiB (32-bit buffer byte offsets)
    if ((long long)L * d * (dtype == FA_F32 ? 4 : 2) >= (1LL << 31)) return FA_ERR_INVALID_ARG;
    if ((long long)B * H > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
    const Tiling t = tiling_dispatch(B * H, L, d, causal, dtype);
    const long long grid = (long long)B * H * ((L + t.br - 1) / t.br);
    if (grid > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// FP8 scores: Q and K as E4M3 codes with block scales, V and O in T
template <class T, int D, bool CAUSAL>
int launch_fp8(const Params& p, hipStream_t stream) {
    const long long grid = (long long)p.BH * p.Tr;
    return fa_detail::launch_kernel(fa_fwd_h_kernel<T, D, CAUSAL, true>, dim3((unsigned)grid),
                                    dim3(HCfg<D, true>::NW * 64), stream, p);
}

template <class T>
int launch_fp8_t(const Params& p, int d, int causal, hipStream_t stream) {
    if (d == 64) return causal ? launch_fp8<T, 64, true>(p, stream) : launch_fp8<T, 64, false>(p, stream);
    return causal ? launch_fp8<T, 128, true>(p, stream) : launch_fp8<T, 128, false>(p, stream);
}

}  // namespace

extern "C" int fa_fwd_fp8(const void* q8, const void* k8, const float* q_scale, const float* k_scale, const void* v,
                          void* o, float* lse, int B, int H, int L, int d, float scale, int causal, int dtype,
                          int block_q, int block_k, hipStream_t stream) {
    if (!q8 || !k8 || !q_scale || !k_scale || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 32 || block_k % 32 != 0) return FA_ERR_INVALID_ARG;
    if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;             // V and O are 16-bit here
    const int rc = check_args(B, H, L, d, causal, dtype);
    if (rc != FA_OK) return rc;
    if (((uintptr_t)q8 | (uintptr_t)k8 | (uintptr_t)v | (uintptr_t)o) % 16 != 0 ||
        ((uintptr_t)lse | (uintptr_t)q_scale | (uintptr_t)k_scale) % 4 != 0)
        return FA_ERR_ALIGN;
    Params p = make_params(q8, k8, v, o, lse, B * H, L, scale, HCfg<128, true>::BR);
    p.qsc = q_scale;
    p.ksc = k_scale;
    p.bq = block_q;
    p.bk = block_k;
    p.nbq = (int)(((long long)L + block_q - 1) / block_q);
    p.nbk = (int)(((long long)L + block_k - 1) / block_k);
    return dtype == FA_BF16 ? launch_fp8_t<__bf16>(p, d, causal, stream) : launch_fp8_t<_Float16>(p, d, causal, stream);
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int L,
                      int d, float scale, int causal, int dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    const int rc = check_args(B, H, L, d, causal, dtype);
    if (rc != FA_OK) return rc;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
    const int BH = B * H;
    if (dtype == FA_BF16) {
        if (d == 64)
            return causal ? launch<__bf16, 64, true>(q, k, v, o, lse, BH, L, scale, stream)
                          : launch<__bf16, 64, false>(q, k, v, o, lse, BH, L, scale, stream);
        return causal ? launch<__bf16, 128, true>(q, k, v, o, lse, BH, L, scale, stream)
                      : launch<__bf16, 128, false>(q, k, v, o, lse, BH, L, scale, stream);
    }
    if (dtype == FA_F16) {
        if (d == 64)
            return causal ? launch<_Float16, 64, true>(q, k, v, o, lse, BH, L, scale, stream)
                          : launch<_Float16, 64, false>(q, k, v, o, lse, BH, L, scale, stream);
        return causal ? launch<_Float16, 128, true>(q, k, v, o, lse, BH, L, scale, stream)
                      : launch<_Float16, 128, false>(q, k, v, o, lse, BH, L, scale, stream);
    }
    if (d == 64)
        return causal ? launch<float, 64, true>(q, k, v, o, lse, BH, L, scale, stream)
                      : launch<float, 64, false>(q, k, v, o, lse, BH, L, scale, stream);
    return causal ? launch<float, 128, true>(q, k, v, o, lse, BH, L, scale, stream)
                  : launch<float, 128, false>(q, k, v, o, lse, BH, L, scale, stream);
}

extern "C" const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK:
            return "success";
        case FA_ERR_INVALID_ARG:
            return "invalid argument (null pointer, non-positive size, bad scale or causal flag, or size overflow)";
        case FA_ERR_UNSUPPORTED:
            return "unsupported head dimension (64 or 128) or dtype (0 f32, 1 f16, 2 bf16)";
        case FA_ERR_ALIGN:
            return "misaligned pointer (q, k, v, o need 16 bytes; lse needs 4)";
        case FA_ERR_HIP:
            return "a HIP call failed (see fa_last_hip_error)";
        case FA_ERR_SCRATCH:
            return "the partial results exceed the library's no-allocation scratch (FA_NOALLOC_SCRATCH_BYTES)";
        default:
            return "unknown status";
    }
}

extern "C" int fa_last_hip_error(void) { return fa_detail::g_last_hip; }

extern "C" int fa_fwd_tiling(int B, int H, int L, int d, int causal, int dtype, int* block_rows, int* block_cols,
                             long long* workgroups) {
    const int rc = check_args(B, H, L, d, causal, dtype);
    if (rc != FA_OK) return rc;
    const Tiling t = tiling_dispatch(B * H, L, d, causal, dtype);
    if (block_rows) *block_rows = t.br;
    if (block_cols) *block_cols = t.bc;
    if (workgroups) *workgroups = (long long)B * H * ((L + t.br - 1) / t.br);
    return FA_OK;
}
