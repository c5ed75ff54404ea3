/*
 * fp64 CPU oracle for the exact attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the tests, the smoke check and the CPU-baseline leg of
 * the bench use it.  It shares no code with the GPU library.
 *
 * What it computes is the plain definition of attention, not the tiled
 * algorithm, because the tiled online-softmax method reaches exactly that
 * result ("FlashAttention 深度解析", first article, section 3.4: the
 * induction over K/V blocks; "FlashAttention: как реально считается attention
 * на GPU": the tiled pass computes the same thing as ordinary attention).
 * Per (batch, head) and query row i, in float64, from the stored inputs
 * widened exactly:
 *     s_ij  = scale * (q_i . k_j)            (j > i is -inf when causal)
 *     m_i   = max_j s_ij
 *     p_ij  = exp(s_ij - m_i)                (safe softmax, two passes)
 *     l_i   = sum_j p_ij
 *     o_i   = (sum_j p_ij v_j) / l_i
 *     lse_i = m_i + ln(l_i)
 * (standard attention: "FlashAttention 深度解析" first article section 2.3;
 * safe softmax: "大语言模型研究14" section 1.1; logsumexp:
 * "04 Transformers, Attention, and FlashAttention", FlashAttention-2
 * Algorithm 1, the statistic L_i = m_i + log l_i.)
 */
#ifndef FA_ORACLE_H
#define FA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* storage type codes of q, k, v: 0 = float32, 1 = IEEE binary16, 2 = bfloat16,
 * 3 = float64 (float64 exists for the oracle's own pins; the GPU library has
 * no float64 path) */
enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_F64 = 3 };

/*
 * q, k, v : host arrays (B, H, L, d), row-major, d fastest, in the storage type.
 * rows    : host array of `nrows` query indices in [0, L) checked per (b, h);
 *           NULL means every row (then nrows must equal L).
 * o       : host float64 (B, H, nrows, d);  lse : host float64 (B, H, nrows).
 * nthreads: OpenMP threads over rows (<= 0: the OpenMP default).
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int fa_oracle_fwd(const void* q, const void* k, const void* v, int dtype,
                  int B, int H, int L, int d, double scale, int causal,
                  const int* rows, int nrows, double* o, double* lse, int nthreads);

/*
 * Brute-force twin for tiny shapes: float64 inputs (B, H, L, d), and every
 * score is recomputed from q and k wherever it is used (O(L^2 d^2)).
 * Shares no helper with fa_oracle_fwd.  Returns 0, or -1 on a bad argument.
 */
int fa_oracle_brute(const double* q, const double* k, const double* v,
                    int B, int H, int L, int d, double scale, int causal,
                    double* o, double* lse);

/*
 * Attention of Lq query rows against the keys [kv_begin, kv_end) of a head
 * with Lk keys (no mask): the same definition as fa_oracle_fwd on a
 * rectangular score block.  This is one K/V block's task in Flash-Decoding
 * ("04 Transformers, Attention, and FlashAttention", the Flash Decoding
 * steps: split K/V into blocks, run each as a small attention task, merge).
 * q : (B, H, Lq, d); k, v : (B, H, Lk, d), storage type `dtype`.
 * o : float64 (B, H, Lq, d); lse : float64 (B, H, Lq).
 * An empty range (kv_begin == kv_end) has no keys: l = 0, so by convention
 * o = 0 and lse = -inf (the neutral element of the merge below).
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int fa_oracle_range(const void* q, const void* k, const void* v, int dtype,
                    int B, int H, int Lq, int Lk, int d, double scale,
                    int kv_begin, int kv_end, double* o, double* lse, int nthreads);

/*
 * Merge of attention results over disjoint key sets (the third Flash
 * Decoding step).  For each of n rows, part s holds its normalised output
 * o_s (d values) and lse_s = m_s + ln l_s.  The pages' rescale rule
 * (running max m, sum rescaled by exp(m_old - m_new), "FlashAttention
 * 深度解析" first article, online softmax) applied to the parts gives
 *     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s,
 * evaluated here with the largest lse_s as the shift.  Parts with
 * lse_s = -inf contribute nothing; if every part is empty, o = 0 and
 * lse = -inf.
 * o_parts : float64 (nsplit, n, d); lse_parts : float64 (nsplit, n).
 * o : float64 (n, d); lse : float64 (n).  Returns 0, or -1 on a bad argument.
 */
int fa_oracle_merge(const double* o_parts, const double* lse_parts, int nsplit, int n, int d,
                    double* o, double* lse);

/*
 * Gradients of attention with respect to q, k and v for an upstream gradient
 * dO of the output ("FlashAttention 深度解析", first article, section 4.1):
 *     P   = softmax_rows(S),   S = scale * Q K^T (causal: key j > query i is -inf)
 *     dV  = P^T dO
 *     dP  = dO V^T
 *     dS  = dP (.) P - P (.) (sum_j dP_ij P_ij)      (row-wise sum)
 *     dQ  = scale * dS K,      dK = scale * dS^T Q
 * (dQ and dK are the chain rule through S = scale * Q K^T.)  P is formed here
 * from the definition in float64; the GPU recomputes it from the stored lse.
 * q, k, v, dout : host (B, H, L, d) in the storage type `dtype`.
 * dq, dk, dv    : host float64 (B, H, L, d).  Returns 0, or -1 on a bad
 * argument (nothing written).  Cost O(L^2 d) per head, OpenMP over rows.
 */
int fa_oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                  int B, int H, int L, int d, double scale, int causal,
                  double* dq, double* dk, double* dv, int nthreads);

/*
 * FP8 block quantisation ("FlashAttention 深度解析", third article
 * (FlashAttention-3), section 2.3): Q and K are cut into blocks, each block is scaled
 * into the FP8 range on its own, s = max|block| / FP8_MAX and
 * X_FP8 = Quantize(X_block / s), and the scores are dequantised after the
 * product: S = (Q_FP8 K_FP8^T) * s_q * s_k * scale.
 *
 * The format is E4M3 as the OCP 8-bit floating point specification defines
 * it: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits, exponent field 0
 * for zero and subnormals (fraction/8 * 2^-6), no infinities, S.1111.111 the
 * only NaN, so the largest finite value (FP8_MAX) is 1.75 * 2^8 = 448.
 */

/* Value of an E4M3 code (0..255); NaN for the NaN codes and out-of-range codes. */
double fa_oracle_e4m3_value(int code);

/* E4M3 code of a finite float with |x| <= 448, rounded to nearest, ties to
 * even (the even code is the one whose last fraction bit is 0); -0.0 gives
 * 0x80.  Returns -1 for NaN or |x| > 448. */
int fa_oracle_e4m3_code(float x);

/*
 * Quantise x (B, H, L, d) in blocks of `block` consecutive rows of one
 * (b, h) (the last block of a head may be short), all d columns of a row in
 * its block.  Per block, in float32: amax = max |x|; s = amax / 448 (s = 1
 * for an all-zero block); each element's code is e4m3_code(clamp(x / s,
 * -448, 448)) (the clamp only absorbs the rounding of s).
 * x8 : (B, H, L, d) codes; scales : float32 (B*H, ceil(L / block)).
 * dtype: float32, float16 or bfloat16 storage.  Returns 0, or -1 on a bad
 * argument.
 */
int fa_oracle_quantize_fp8(const void* x, int dtype, int B, int H, int L, int d, int block,
                           unsigned char* x8, float* scales);

/*
 * Attention on block-quantised Q and K: the definition of fa_oracle_fwd with
 * q_ic = e4m3_value(q8_ic) * q_scale[bh][i / block_q] and
 * k_jc = e4m3_value(k8_jc) * k_scale[bh][j / block_k] (both exact in
 * float64), v widened from its storage type.
 * q8, k8 : (B, H, L, d) codes; q_scale : (B*H, ceil(L/block_q));
 * k_scale : (B*H, ceil(L/block_k)); rows, o, lse as for fa_oracle_fwd.
 */
int fa_oracle_fwd_fp8(const unsigned char* q8, const unsigned char* k8, const float* q_scale, const float* k_scale,
                      const void* v, int dtype, int B, int H, int L, int d, double scale, int causal,
                      int block_q, int block_k, const int* rows, int nrows, double* o, double* lse, int nthreads);

/* Threads an fa_oracle_fwd call with nthreads <= 0 would use. */
int fa_oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
