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

int fa_oracle_fwd(const void* q, const void* k, const void* v, int dtype,
                  int B, int H, int L, int d, double scale, int causal,
                  const int* rows, int nrows, double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o || !lse) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return -1;
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || nrows <= 0) return -1;
    if (causal != 0 && causal != 1) return -1;
    if (!rows && nrows != L) return -1;
    if (rows) {
        for (int r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= L) return -1;
    }
    if (nthreads <= 0) nthreads = fa_oracle_max_threads();

    const size_t head = (size_t)L * (size_t)d;
    double* kd = (double*)malloc(head * sizeof(double));
    double* vd = (double*)malloc(head * sizeof(double));
    if (!kd || !vd) {
        free(kd);
        free(vd);
        return -1;
    }

    for (int bh = 0; bh < B * H; ++bh) {
        const size_t base = (size_t)bh * head;
        for (size_t e = 0; e < head; ++e) {
            kd[e] = widen(k, dtype, base + e);
            vd[e] = widen(v, dtype, base + e);
        }
#pragma omp parallel num_threads(nthreads)
        {
            double* qi = (double*)malloc((size_t)d * sizeof(double));
            double* s = (double*)malloc((size_t)L * sizeof(double));
            double* p = (double*)malloc((size_t)L * sizeof(double));
#pragma omp for schedule(dynamic, 1)
            for (int r = 0; r < nrows; ++r) {
                const int i = rows ? rows[r] : r;
                for (int c = 0; c < d; ++c) qi[c] = widen(q, dtype, base + (size_t)i * d + c);

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
                double* oi = o + ((size_t)bh * nrows + r) * d;
                for (int c = 0; c < d; ++c) oi[c] = 0.0;
                for (int j = 0; j < L; ++j) {
                    const double* vj = vd + (size_t)j * d;
                    for (int c = 0; c < d; ++c) oi[c] += p[j] * vj[c];
                }
                for (int c = 0; c < d; ++c) oi[c] /= l;
                lse[(size_t)bh * nrows + r] = m + log(l);
            }
            free(qi);
            free(s);
            free(p);
        }
    }
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
