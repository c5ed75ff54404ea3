/*
 * fa.h -- exact attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; no C++ or framework types cross it.
 *
 * Operation (per batch b and head h, on one GPU):
 *     S   = scale * Q K^T                      (L x L, never materialised)
 *     S_ij = -inf for key j > query i          (only when causal = 1)
 *     O   = softmax_rows(S) V                  (L x d)
 *     lse_i = max_j S_ij + ln sum_j exp(S_ij - max_j S_ij)
 * The definition is standard attention ("FlashAttention 深度解析", first
 * article, section 2.3) with the causal mask of its second article, section
 * 2.3 (a query attends to keys at or before its own position), and the
 * logsumexp statistic L_i = m_i + log l_i that FlashAttention-2 Algorithm 1
 * writes next to O ("04 Transformers, Attention, and FlashAttention").
 * It is computed with the tiled online-softmax recurrence of that algorithm
 * (running max m, running sum l, unnormalised output rescaled by
 * exp(m_old - m_new) per K/V block, one division by l at the end), which is
 * exact: the result equals the definition up to floating-point rounding.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, k, v and o.  lse is always float32. */
enum fa_dtype {
    FA_F32 = 0,   /* IEEE binary32; the products and P stay in fp32       */
    FA_F16 = 1,   /* IEEE binary16; fp32 accumulation, P rounded to fp16  */
    FA_BF16 = 2   /* bfloat16;      fp32 accumulation, P rounded to bf16  */
};

/* Return codes.  0 is success; every failure is negative. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,  /* null pointer; B, H or L <= 0; scale not finite or <= 0;
                                 causal not 0/1; B*H*L*d >= 2^62; too many Q tiles for one grid */
    FA_ERR_UNSUPPORTED = -2,  /* d not 64 or 128; unknown dtype                              */
    FA_ERR_ALIGN = -3,        /* q, k, v or o not 16-byte aligned; lse not 4-byte aligned   */
    FA_ERR_HIP = -4,          /* a HIP call failed; see fa_last_hip_error()                 */
    FA_ERR_SCRATCH = -5       /* fa_fwd_splitkv_noalloc: the partial results would exceed
                                 FA_NOALLOC_SCRATCH_BYTES                                   */
};

/*
 * fa_fwd -- enqueue the forward pass on `stream` and return.
 *
 * q, k, v : device pointers, read only, each (B, H, L, d) contiguous row-major
 *           with d fastest: element (b, h, l, c) at ((b*H + h)*L + l)*d + c.
 * o       : device pointer, (B, H, L, d) in the same layout and type; fully
 *           overwritten.  Must not overlap q, k, v or lse.
 * lse     : device pointer, float32 (B, H, L) contiguous; fully overwritten
 *           with the natural-log logsumexp of each scaled score row.
 * B, H, L : batch, heads, sequence length (L_q = L_k = L).
 * d       : head dimension, 64 or 128.
 * scale   : multiplies Q K^T before the softmax (1/sqrt(d) in the usual form);
 *           finite and > 0.
 * causal  : 0 = full attention; 1 = key j > query i is masked out.
 * dtype   : an fa_dtype value.
 * stream  : HIP stream (0 = the null stream).
 *
 * Ownership: the caller owns all five buffers.  The library allocates and
 * frees nothing, copies nothing to or from the host, never synchronises, and
 * keeps no state between calls; calls are thread-safe and reentrant.
 * Results are valid once `stream` has reached this work.
 *
 * Errors: argument errors are detected on the host before anything is
 * enqueued (no partial writes) and return FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED or FA_ERR_ALIGN.  A launch failure returns FA_ERR_HIP and
 * records the HIP error code for fa_last_hip_error().  NaN or Inf inputs are
 * not errors: they propagate through the arithmetic.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int L, int d, float scale, int causal, int dtype,
           hipStream_t stream);

/* Static description of a return code (never NULL). */
const char* fa_strerror(int status);

/* HIP error code of the last FA_ERR_HIP returned on the calling thread
 * (hipSuccess if none). */
int fa_last_hip_error(void);

/* Query-tile height B_r and key-tile width B_c that fa_fwd uses for a
 * (d, causal, dtype) combination, and the number of workgroups it launches
 * for (B, H, L).  Returns FA_OK or an argument error as fa_fwd would. */
int fa_fwd_tiling(int B, int H, int L, int d, int causal, int dtype,
                  int* block_rows, int* block_cols, long long* workgroups);

/*
 * ---- Split-K/V attention for few query rows (decoding) ----
 *
 * Flash-Decoding ("04 Transformers, Attention, and FlashAttention", the
 * Flash Decoding steps): with only a handful of query rows per head there is
 * not enough query parallelism, so the keys of each (batch, head) are cut into
 * nsplit contiguous chunks, each chunk is attended to as its own small
 * attention task (partial output O_s, normalised by its own sum, and its
 * logsumexp lse_s), and the chunks are merged with the online-softmax rescale
 * rule ("FlashAttention 深度解析", first article: statistics brought to a
 * common maximum by exp(m_old - m_new) and added):
 *     lse = ln sum_s exp(lse_s),    O = sum_s exp(lse_s - lse) O_s.
 * The result is the same attention as fa_fwd with causal = 0, for a query
 * block of Lq rows against Lk keys: the softmax over all Lk keys.
 */

/*
 * fa_splitkv_splits -- the nsplit that fa_fwd_splitkv uses when passed
 * nsplit <= 0: chunks for about 2048 wavefronts in all (a multiple of 4 when
 * above 4), at least 256 keys each.  Returns 0 for non-positive sizes.
 */
int fa_splitkv_splits(int B, int H, int Lk);

/*
 * fa_splitkv_workspace_bytes -- device workspace fa_fwd_splitkv needs for
 * these sizes (nsplit <= 0: the automatic choice).  Returns 0 for
 * non-positive sizes or d not 64/128.
 */
size_t fa_splitkv_workspace_bytes(int B, int H, int Lq, int Lk, int d, int nsplit);

/*
 * fa_fwd_splitkv -- enqueue split-K/V attention and the merge on `stream`.
 *
 * q, o    : device, (B, H, Lq, d) contiguous row-major, d fastest; o fully
 *           overwritten with the attention output in the storage type.
 * k, v    : device, (B, H, Lk, d) in the same layout and type; read only.
 * lse     : device float32 (B, H, Lq); fully overwritten (natural log).
 * Lq      : query rows per (b, h), 1..8 (more rows: use fa_fwd).
 * Lk      : keys per (b, h), 1 .. 2^30.  No mask: every query sees every key.
 * d, scale, dtype : as for fa_fwd.
 * nsplit  : chunks per (b, h); <= 0 picks fa_splitkv_splits(B, H, Lk).
 *           Chunk s covers keys [s*c, min((s+1)*c, Lk)) with c = ceil(Lk/nsplit);
 *           chunks past the end are empty and merge as no contribution.
 * workspace, workspace_size : device scratch of at least
 *           fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit) bytes,
 *           256-byte aligned, owned by the caller; it holds the partial results
 *           (float32 O_s (nsplit, B, H, Lq, d), then float32 lse_s
 *           (nsplit, B, H, Lq), each padded to 256 bytes) until the merge on
 *           the same stream has read them.  Calls sharing a workspace must be
 *           ordered on one stream.
 * The arithmetic is fp32 throughout (no rounding of P), and the output is
 * rounded once to the storage type.
 * Ownership, asynchrony and errors as for fa_fwd.  Lq > 8 returns
 * FA_ERR_UNSUPPORTED; a small workspace, B*H > 65535 or nsplit > 262140
 * returns FA_ERR_INVALID_ARG; a workspace not 256-byte aligned returns
 * FA_ERR_ALIGN.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int dtype, int nsplit,
                   void* workspace, size_t workspace_size, hipStream_t stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * around the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments (minus workspace and workspace_size), same kernels and
 * bit-identical results as fa_fwd_splitkv.  The partial results live in a
 * device array of FA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU
 * it runs on, from that GPU's first call until the process ends.  The GPU is
 * the stream's (the current device for the null stream); the first call on a
 * GPU looks the array's address up (hipGetSymbolAddress, with that GPU made
 * current for the lookup and the caller's current device restored).  The call
 * makes no hipMalloc, hipFree or other allocating call.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on a GPU
 * (different streams, or different host threads, without ordering between
 * them) race and give undefined results.  Calls ordered on one stream are
 * safe.  Nothing in the array needs clearing between calls: every call writes
 * each partial result before its merge reads it.
 *
 * Errors as for fa_fwd_splitkv; FA_ERR_SCRATCH when
 * fa_splitkv_workspace_bytes(B, H, Lq, Lk, d, nsplit) > FA_NOALLOC_SCRATCH_BYTES
 * (pass a smaller nsplit, or use fa_fwd_splitkv); FA_ERR_HIP when the stream's
 * device or the array's address cannot be obtained.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Lq, int Lk, int d, float scale, int dtype, int nsplit,
                           hipStream_t stream);

/*
 * fa_combine -- enqueue only the merge of nsplit partial results.
 *
 * o_part   : device float32 (nsplit, B, H, Lq, d): normalised partial outputs.
 * lse_part : device float32 (nsplit, B, H, Lq): their logsumexp; -inf marks a
 *            part with no keys (its o_part row is ignored).
 * o        : device (B, H, Lq, d) in `dtype`; lse : device float32 (B, H, Lq).
 *            A row whose parts are all empty gets o = 0 and lse = -inf.
 * Lq here may be any positive count (the merge is per row).  Ownership,
 * asynchrony and errors as for fa_fwd (o 16-byte aligned, the float arrays
 * 4-byte aligned).
 */
int fa_combine(const float* o_part, const float* lse_part, int nsplit, int B, int H, int Lq, int d,
               void* o, float* lse, int dtype, hipStream_t stream);

/*
 * ---- Backward pass (gradients with respect to q, k, v) ----
 *
 * For an upstream gradient dO of the output of fa_fwd ("FlashAttention
 * 深度解析", first article, section 4.1: dV = P^T dO, dP = dO V^T,
 * dS = dP (.) P - P (.) rowsum(dP (.) P); dQ = scale dS K and dK = scale dS^T Q
 * by the chain rule through S = scale Q K^T), with P recomputed from q, k and
 * the lse of the forward pass rather than stored ("Recomputation": "04
 * Transformers, Attention, and FlashAttention").  rowsum(dP (.) P)_i is taken
 * as dO_i . O_i, which equals it because O_i = sum_j P_ij V_j.
 */

/* fa_bwd_workspace_bytes -- device workspace fa_bwd needs (B*H*L floats,
 * rounded up to 256 bytes); 0 for non-positive sizes. */
size_t fa_bwd_workspace_bytes(int B, int H, int L);

/*
 * fa_bwd -- enqueue the backward pass on `stream`.
 *
 * q, k, v : the forward pass's inputs; o, lse : its outputs (o in the storage
 *           type, lse float32 (B, H, L)); dout : dO, (B, H, L, d).  All read only.
 * dq, dk, dv : device, (B, H, L, d) in the storage type; fully overwritten
 *           (fp32 accumulation, one rounding at the end).
 * Layouts, B, H, L, d, scale and causal as for fa_fwd; dtype FA_F16 or
 * FA_BF16 (FA_F32 returns FA_ERR_UNSUPPORTED).
 * workspace, workspace_size : caller-owned device scratch of at least
 *           fa_bwd_workspace_bytes(B, H, L) bytes, 256-byte aligned; it holds
 *           D = rowsum(dO (.) O) until the kernels on `stream` have read it.
 * Ownership, asynchrony and errors as for fa_fwd (all tensors 16-byte
 * aligned, lse 4-byte aligned); B*H*ceil(L/128) > 2^31 - 1 or
 * L*d*2 >= 2^31 returns FA_ERR_INVALID_ARG.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int H, int L, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_size, hipStream_t stream);

/*
 * ---- FP8 block-quantised forward pass ----
 *
 * "FlashAttention 深度解析", third article (FlashAttention-3), section 2.3:
 * Q and K are cut into blocks, each block is scaled into the E4M3 range on
 * its own, s = max|block| / 448 and codes = Quantize(block / s), and the
 * scores are dequantised after the product:
 *     S_ij = scale * s_q(block of i) * s_k(block of j) * (q8_i . k8_j)
 * where q8_i, k8_j are the E4M3 values of the codes.  The rest is fa_fwd's
 * operation with this S (mask, softmax, O = P V, lse).  V and O stay 16-bit
 * (the section gives the quantisation for Q and K only).
 *
 * E4M3 is the OCP 8-bit floating point format: 1 sign, 4 exponent (bias 7)
 * and 3 fraction bits, no infinities, largest finite value 448.
 */

/*
 * fa_quantize_fp8 -- enqueue block quantisation of x on `stream`.
 *
 * x      : device, read only, (B, H, L, d) in `dtype` (FA_F16 or FA_BF16),
 *          layout as for fa_fwd; finite values.
 * block  : rows per block (>= 1).  A block is `block` consecutive rows of
 *          one (b, h), all d columns; the last block of a head may be short.
 * x8     : device, (B, H, L, d) bytes, fully overwritten with E4M3 codes:
 *          code = E4M3(clamp(x / s, -448, 448)), round to nearest even, with
 *          the float32 quotient of x by its block's s.
 * scales : device float32 (B*H, ceil(L/block)), fully overwritten:
 *          s = amax / 448 in float32, amax = max |x| over the block; s = 1
 *          for an all-zero block.
 * Ownership, asynchrony and errors as for fa_fwd: x and x8 16-byte aligned,
 * scales 4-byte aligned; d not 64/128 or dtype not 16-bit returns
 * FA_ERR_UNSUPPORTED; block < 1 or B*H > 65535 returns FA_ERR_INVALID_ARG.
 */
int fa_quantize_fp8(const void* x, int dtype, int B, int H, int L, int d, int block, void* x8,
                    float* scales, hipStream_t stream);

/*
 * fa_fwd_fp8 -- enqueue the FP8 forward pass on `stream`.
 *
 * q8, k8  : device, read only, (B, H, L, d) E4M3 codes (as fa_quantize_fp8
 *           writes them).
 * q_scale : device float32 (B*H, ceil(L/block_q)); k_scale : device float32
 *           (B*H, ceil(L/block_k)); finite and > 0.
 * v       : device, read only, (B, H, L, d) in `dtype`.
 * o, lse  : outputs as for fa_fwd (o in `dtype`).
 * block_q : query rows per q_scale block (>= 1); block_k : key rows per
 *           k_scale block, a multiple of 32 (one scale per 32-key MFMA
 *           block).
 * B, H, L, d, scale, causal as for fa_fwd; dtype FA_F16 or FA_BF16
 * (FA_F32 returns FA_ERR_UNSUPPORTED).
 * Ownership, asynchrony and errors as for fa_fwd: q8, k8, v and o 16-byte
 * aligned, the float arrays 4-byte aligned; a bad block size returns
 * FA_ERR_INVALID_ARG.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const float* q_scale, const float* k_scale, const void* v,
               void* o, float* lse, int B, int H, int L, int d, float scale, int causal, int dtype,
               int block_q, int block_k, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FA_H */
