/*
 * fp64 CPU oracle for the exact attention forward pass (definitions in
 * fa_oracle.h).  TEST INFRASTRUCTURE ONLY: the product library never links
 * or calls this file.  Plain C, no blocking, no fusion: each query row's full
 * score row is materialised, then its maximum, its exponentials, their sum,
 * the weighted sum of V and the logsumexp are computed in that order.
 */
#include "fa_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* exact widening of one stored element to double */
static double widen(const void* base, int dtype, size_t idx) {
    if (dtype == ORACLE_F64) {
        return ((const double*)base)[idx];
    }
    if (dtype == ORACLE_F32) {
        return (double)((const float*)base)[idx];
    }
    if (dtype == ORACLE_BF16) {
        /* bfloat16 is the upper half of a binary32 */
        uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
    uint16_t h = ((const uint16_t*)base)[idx];
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double mag;
    if (ex == 0) {
        mag = ldexp((double)fr, -24);               /* zero or subnormal */
    } else if (ex == 31) {
        mag = fr ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(fr + 1024), ex - 25);  /* (1 + fr/1024) * 2^(ex-15) */
    }
    return sign ? -mag : mag;
}

int fa_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One head: rows `rows` (NULL: all L) of qd against kd, vd, all (L x d)
 * float64.  oh : (nrows x d), lseh : (nrows). */
static void attend_head(const double* qd, const double* kd, const double* vd, int L, int d, double scale,
                        int causal, const int* rows, int nrows, double* oh, double* lseh, int nthreads) {
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc((size_t)L * sizeof(double));
        double* p = (double*)malloc((size_t)L * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            const int i = rows ? rows[r] : r;
            const double* qi = qd + (size_t)i * d;

            /* S row: scale * q_i . k_j ; causal keys after the query are -inf */
            for (int j = 0; j < L; ++j) {
                if (causal && j > i) {
                    s[j] = -INFINITY;
                    continue;
                }
                double dot = 0.0;
                const double* kj = kd + (size_t)j * d;
                for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
                s[j] = scale * dot;
            }
            /* row maximum */
            double m = -INFINITY;
            for (int j = 0; j < L; ++j)
                if (s[j] > m) m = s[j];
            /* exponentials relative to the maximum, and their sum */
            double l = 0.0;
            for (int j = 0; j < L; ++j) {
                p[j] = exp(s[j] - m);
                l += p[j];
            }
            /* O row = (P row . V) / l */
            double* oi = oh + (size_t)r * d;
            for (int c = 0; c < d; ++c) oi[c] = 0.0;
            for (int j = 0; j < L; ++j) {
                const double* vj = vd + (size_t)j * d;
                for (int c = 0; c < d; ++c) oi[c] += p[j] * vj[c];
            }
            for (int c = 0; c < d; ++c) oi[c] /= l;
            lseh[r] = m + log(l);
        }
        free(s);
        free(p);
    }
}

static int check_rows(int L, const int* rows, int nrows) {
    if (nrows <= 0 || (!rows && nrows != L)) return -1;
    if (rows) {
        for (int r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= L) return -1;
    }
    return 0;
}

int fa_oracle_fwd(const void* q, const void* k, const void* v, int dtype,
                  int B, int H, int L, int d, double scale, int causal,
                  const int* rows, int nrows, double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o || !lse) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0) return -1;
    if (causal != 0 && causal != 1) return -1;
    if (check_rows(L, rows, nrows)) return -1;
    if (nthreads <= 0) nthreads = fa_oracle_max_threads();

    const size_t head = (size_t)L * (size_t)d;
    double* qd = (double*)malloc(head * sizeof(double));
    double* kd = (double*)malloc(head * sizeof(double));
    double* vd = (double*)malloc(head * sizeof(double));
    if (!qd || !kd || !vd) {
        free(qd);
        free(kd);
        free(vd);
        return -1;
    }
    for (int bh = 0; bh < B * H; ++bh) {
        const size_t base = (size_t)bh * head;
        for (size_t e = 0; e < head; ++e) {
            qd[e] = widen(q, dtype, base + e);
            kd[e] = widen(k, dtype, base + e);
            vd[e] = widen(v, dtype, base + e);
        }
        attend_head(qd, kd, vd, L, d, scale, causal, rows, nrows, o + (size_t)bh * nrows * d,
                    lse + (size_t)bh * nrows, nthreads);
    }
    free(qd);
    free(kd);
    free(vd);
    return 0;
}

/* ---- brute-force twin: no shared helpers, every score recomputed ---- */

static double brute_score(const double* qh, const double* kh, int d, double scale, int i, int j) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += qh[(size_t)i * d + c] * kh[(size_t)j * d + c];
    return acc * scale;
}

int fa_oracle_brute(const double* q, const double* k, const double* v,
                    int B, int H, int L, int d, double scale, int causal,
                    double* o, double* lse) {
    if (!q || !k || !v || !o || !lse) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0) return -1;
    if (causal != 0 && causal != 1) return -1;
    for (int bh = 0; bh < B * H; ++bh) {
        const size_t off = (size_t)bh * L * d;
        const double* qh = q + off;
        const double* kh = k + off;
        const double* vh = v + off;
        for (int i = 0; i < L; ++i) {
            const int last = causal ? i : L - 1;   /* keys 0..last are visible */
            double mx = -INFINITY;
            for (int j = 0; j <= last; ++j) {
                double sc = brute_score(qh, kh, d, scale, i, j);
                if (sc > mx) mx = sc;
            }
            double den = 0.0;
            for (int j = 0; j <= last; ++j) den += exp(brute_score(qh, kh, d, scale, i, j) - mx);
            for (int c = 0; c < d; ++c) {
                double num = 0.0;
                for (int j = 0; j <= last; ++j)
                    num += exp(brute_score(qh, kh, d, scale, i, j) - mx) * vh[(size_t)j * d + c];
                o[off + (size_t)i * d + c] = num / den;
            }
            lse[(size_t)bh * L + i] = mx + log(den);
        }
    }
    return 0;
}

/* ---- one K/V block's attention, rectangular (Flash-Decoding task) ---- */

int fa_oracle_range(const void* q, const void* k, const void* v, int dtype,
                    int B, int H, int Lq, int Lk, int d, double scale,
                    int kv_begin, int kv_end, double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o || !lse) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || d <= 0) return -1;
    if (kv_begin < 0 || kv_end < kv_begin || kv_end > Lk) return -1;
    if (nthreads <= 0) nthreads = fa_oracle_max_threads();
    const int n = kv_end - kv_begin;

    for (int bh = 0; bh < B * H; ++bh) {
        const size_t qbase = (size_t)bh * Lq * d;
        const size_t kbase = (size_t)bh * Lk * d;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
        for (int i = 0; i < Lq; ++i) {
            double* oi = o + qbase + (size_t)i * d;
            for (int c = 0; c < d; ++c) oi[c] = 0.0;
            if (n == 0) {
                lse[(size_t)bh * Lq + i] = -INFINITY;
                continue;
            }
            double* s = (double*)malloc((size_t)n * sizeof(double));
            /* score row over the block's keys */
            for (int j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += widen(q, dtype, qbase + (size_t)i * d + c) *
                           widen(k, dtype, kbase + (size_t)(kv_begin + j) * d + c);
                s[j] = scale * dot;
            }
            double m = -INFINITY;
            for (int j = 0; j < n; ++j)
                if (s[j] > m) m = s[j];
            double l = 0.0;
            for (int j = 0; j < n; ++j) {
                s[j] = exp(s[j] - m); /* s now holds p */
                l += s[j];
            }
            for (int j = 0; j < n; ++j)
                for (int c = 0; c < d; ++c) oi[c] += s[j] * widen(v, dtype, kbase + (size_t)(kv_begin + j) * d + c);
            for (int c = 0; c < d; ++c) oi[c] /= l;
            lse[(size_t)bh * Lq + i] = m + log(l);
            free(s);
        }
    }
    return 0;
}

/* ---- merge of per-block results ---- */

int fa_oracle_merge(const double* o_parts, const double* lse_parts, int nsplit, int n, int d,
                    double* o, double* lse) {
    if (!o_parts || !lse_parts || !o || !lse) return -1;
    if (nsplit <= 0 || n <= 0 || d <= 0) return -1;
    for (int r = 0; r < n; ++r) {
        double mx = -INFINITY;
        for (int t = 0; t < nsplit; ++t) {
            const double x = lse_parts[(size_t)t * n + r];
            if (x > mx) mx = x;
        }
        double* orow = o + (size_t)r * d;
        for (int c = 0; c < d; ++c) orow[c] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int t = 0; t < nsplit; ++t) wsum += exp(lse_parts[(size_t)t * n + r] - mx);
        const double total = mx + log(wsum);
        for (int t = 0; t < nsplit; ++t) {
            const double w = exp(lse_parts[(size_t)t * n + r] - total);
            const double* op = o_parts + ((size_t)t * n + r) * d;
            for (int c = 0; c < d; ++c) orow[c] += w * op[c];
        }
        lse[r] = total;
    }
    return 0;
}

/* ---- gradients (definition in float64, P materialised per head) ---- */

int fa_oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                  int B, int H, int L, int d, double scale, int causal,
                  double* dq, double* dk, double* dv, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0) return -1;
    if (causal != 0 && causal != 1) return -1;
    if (nthreads <= 0) nthreads = fa_oracle_max_threads();
    const size_t head = (size_t)L * d;
    double* qd = (double*)malloc(head * sizeof(double));
    double* kd = (double*)malloc(head * sizeof(double));
    double* vd = (double*)malloc(head * sizeof(double));
    double* gd = (double*)malloc(head * sizeof(double));
    double* P = (double*)malloc((size_t)L * L * sizeof(double));
    double* dS = (double*)malloc((size_t)L * L * sizeof(double));
    if (!qd || !kd || !vd || !gd || !P || !dS) {
        free(qd); free(kd); free(vd); free(gd); free(P); free(dS);
        return -1;
    }
    for (int bh = 0; bh < B * H; ++bh) {
        const size_t base = (size_t)bh * head;
        for (size_t e = 0; e < head; ++e) {
            qd[e] = widen(q, dtype, base + e);
            kd[e] = widen(k, dtype, base + e);
            vd[e] = widen(v, dtype, base + e);
            gd[e] = widen(dout, dtype, base + e);
        }
        /* per query row: P row (softmax of the scaled scores), dP row, dS row */
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4)
        for (int i = 0; i < L; ++i) {
            double* p = P + (size_t)i * L;
            double* ds = dS + (size_t)i * L;
            double m = -INFINITY;
            for (int j = 0; j < L; ++j) {
                if (causal && j > i) {
                    p[j] = -INFINITY;
                    continue;
                }
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qd[(size_t)i * d + c] * kd[(size_t)j * d + c];
                p[j] = scale * dot;
                if (p[j] > m) m = p[j];
            }
            double l = 0.0;
            for (int j = 0; j < L; ++j) {
                p[j] = exp(p[j] - m);
                l += p[j];
            }
            for (int j = 0; j < L; ++j) p[j] /= l;
            /* dP_ij = dO_i . V_j, and the row sum of dP (.) P */
            double rs = 0.0;
            for (int j = 0; j < L; ++j) {
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += gd[(size_t)i * d + c] * vd[(size_t)j * d + c];
                ds[j] = dot;
                rs += dot * p[j];
            }
            for (int j = 0; j < L; ++j) ds[j] = p[j] * (ds[j] - rs);
            /* dQ_i = scale * sum_j dS_ij K_j */
            double* gq = dq + base + (size_t)i * d;
            for (int c = 0; c < d; ++c) gq[c] = 0.0;
            for (int j = 0; j < L; ++j)
                for (int c = 0; c < d; ++c) gq[c] += ds[j] * kd[(size_t)j * d + c];
            for (int c = 0; c < d; ++c) gq[c] *= scale;
        }
        /* per key row: dV_j = sum_i P_ij dO_i, dK_j = scale * sum_i dS_ij Q_i */
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4)
        for (int j = 0; j < L; ++j) {
            double* gv = dv + base + (size_t)j * d;
            double* gk = dk + base + (size_t)j * d;
            for (int c = 0; c < d; ++c) {
                gv[c] = 0.0;
                gk[c] = 0.0;
            }
            for (int i = 0; i < L; ++i) {
                const double pij = P[(size_t)i * L + j];
                const double sij = dS[(size_t)i * L + j];
                for (int c = 0; c < d; ++c) {
                    gv[c] += pij * gd[(size_t)i * d + c];
                    gk[c] += sij * qd[(size_t)i * d + c];
                }
            }
            for (int c = 0; c < d; ++c) gk[c] *= scale;
        }
    }
    free(qd); free(kd); free(vd); free(gd); free(P); free(dS);
    return 0;
}

/* ---- FP8 (E4M3) block quantisation and attention on the quantised Q, K ---- */

double fa_oracle_e4m3_value(int code) {
    if (code < 0 || code > 255) return NAN;
    const int sign = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    if (ex == 15 && man == 7) return NAN;
    /* exponent field 0: subnormal man/8 * 2^-6; else (1 + man/8) * 2^(ex-7) */
    const double mag = ex == 0 ? ldexp((double)man, -9) : ldexp((double)(8 + man), ex - 10);
    return sign ? -mag : mag;
}

int fa_oracle_e4m3_code(float x) {
    if (!(fabsf(x) <= 448.0f)) return -1;       /* NaN or out of range */
    const int sign = signbit(x) ? 1 : 0;
    const double a = fabs((double)x);
    if (a == 0.0) return sign << 7;
    int e2;
    (void)frexp(a, &e2);                        /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                             /* a = 1.x * 2^e */
    if (e < -6) e = -6;                         /* subnormals share the quantum of the smallest binade */
    const double quantum = ldexp(1.0, e - 3);   /* 3 fraction bits */
    double m = nearbyint(a / quantum);          /* exact quotient; ties to even (default rounding mode) */
    /* m counts quanta: [8, 16] in a normal binade, [0, 8] in the subnormal one */
    if (m >= 16.0) {                            /* rounded up into the next binade */
        m = 8.0;
        e += 1;
    }
    int code;
    if (m < 8.0) {
        code = (int)m;                          /* subnormal: exponent field 0 */
    } else {
        code = ((e + 7) << 3) | ((int)m - 8);
    }
    return (sign << 7) | code;
}

int fa_oracle_quantize_fp8(const void* x, int dtype, int B, int H, int L, int d, int block,
                           unsigned char* x8, float* scales) {
    if (!x || !x8 || !scales) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || block <= 0) return -1;
    const int nblk = (L + block - 1) / block;
    for (int bh = 0; bh < B * H; ++bh) {
        for (int b = 0; b < nblk; ++b) {
            const int r0 = b * block, r1 = r0 + block < L ? r0 + block : L;
            const size_t e0 = ((size_t)bh * L + r0) * d, e1 = ((size_t)bh * L + r1) * d;
            /* amax over the block (the stored values are exact in float32) */
            float amax = 0.0f;
            for (size_t e = e0; e < e1; ++e) {
                const float a = fabsf((float)widen(x, dtype, e));
                if (a > amax) amax = a;
            }
            /* s = amax / 448 in float32; an all-zero block takes s = 1 */
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[(size_t)bh * nblk + b] = s;
            for (size_t e = e0; e < e1; ++e) {
                float y = (float)widen(x, dtype, e) / s;     /* float32 quotient */
                if (y > 448.0f) y = 448.0f;
                if (y < -448.0f) y = -448.0f;
                x8[e] = (unsigned char)fa_oracle_e4m3_code(y);
            }
        }
    }
    return 0;
}

int fa_oracle_fwd_fp8(const unsigned char* q8, const unsigned char* k8, const float* q_scale, const float* k_scale,
                      const void* v, int dtype, int B, int H, int L, int d, double scale, int causal,
                      int block_q, int block_k, const int* rows, int nrows, double* o, double* lse, int nthreads) {
    if (!q8 || !k8 || !q_scale || !k_scale || !v || !o || !lse) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || block_q <= 0 || block_k <= 0) return -1;
    if (causal != 0 && causal != 1) return -1;
    if (check_rows(L, rows, nrows)) return -1;
    if (nthreads <= 0) nthreads = fa_oracle_max_threads();
    const int nbq = (L + block_q - 1) / block_q, nbk = (L + block_k - 1) / block_k;
    const size_t head = (size_t)L * (size_t)d;
    double* qd = (double*)malloc(head * sizeof(double));
    double* kd = (double*)malloc(head * sizeof(double));
    double* vd = (double*)malloc(head * sizeof(double));
    if (!qd || !kd || !vd) {
        free(qd);
        free(kd);
        free(vd);
        return -1;
    }
    for (int bh = 0; bh < B * H; ++bh) {
        const size_t base = (size_t)bh * head;
        /* dequantise: code value times its block's scale (exact in float64:
         * 4 significant bits times 24) */
        for (int i = 0; i < L; ++i) {
            const double sq = q_scale[(size_t)bh * nbq + i / block_q];
            const double sk = k_scale[(size_t)bh * nbk + i / block_k];
            for (int c = 0; c < d; ++c) {
                const size_t e = (size_t)i * d + c;
                qd[e] = fa_oracle_e4m3_value(q8[base + e]) * sq;
                kd[e] = fa_oracle_e4m3_value(k8[base + e]) * sk;
                vd[e] = widen(v, dtype, base + e);
            }
        }
        attend_head(qd, kd, vd, L, d, scale, causal, rows, nrows, o + (size_t)bh * nrows * d,
                    lse + (size_t)bh * nrows, nthreads);
    }
    free(qd);
    free(kd);
    free(vd);
    return 0;
}
