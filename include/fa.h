/*
 * fa.h — C ABI of the exact tiled attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,   L = per-row logsumexp,
 * and its gradients, tile by tile with online softmax in the FlashAttention-2
 * order: one workgroup per Q tile (page "6.2 FlashAttention V2 chi tiết",
 * sections 2.2 and 6.1), K/V tiles streamed through LDS, an unnormalised output
 * rescaled only by exp(m_old - m_new) and divided once at the end (section
 * 3.2), causal tiles above the diagonal skipped (section 5.3), and a backward
 * pass in two launches (section 7.2; CSDN FlashAttention-2 article,
 * "并行性 / 反向传播"): a Q-outer pass that forms D = rowsum(dO o O) and
 * writes dQ once, then workgroups that each own one K/V column block and
 * write dK, dV once; no atomics, deterministic. fa_bwd_atomic is the
 * single-pass variant that adds dQ with fp32 atomics after a D preprocess.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA memory)
 *    on the device that is current when the call is made.
 *  - Layout is contiguous row-major "BHSD": Q, O, dO, dQ are
 *    [batch][n_q_heads][seqlen_q][head_dim]; K, V, dK, dV are
 *    [batch][n_kv_heads][seqlen_k][head_dim]; L (lse) and D are
 *    [batch][n_q_heads][seqlen_q].
 *  - Grouped-query attention: G = n_q_heads / n_kv_heads query heads share one
 *    K/V head, and query head h uses K/V head h / G (contiguous groups; the
 *    CSDN article, "多查询注意力和分组查询注意力").
 *  - Base pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it; the call returns without synchronising.
 *  - Ownership: the caller allocates and frees every buffer and owns the
 *    stream. The library never allocates, frees or synchronises, and keeps no
 *    state between calls except a thread-local error message; a call only
 *    enqueues kernels, so fa_fwd and fa_bwd can be captured into a HIP graph
 *    on a capturing stream and replayed.
 *  - Errors: argument problems are detected on the host before anything is
 *    enqueued, and leave every output untouched. A launch failure returns
 *    FA_ERR_HIP. Faults inside a kernel surface at the caller's next
 *    synchronisation, as usual for HIP.
 *  - Numerics: fp32 accumulation; probabilities P (and in the backward dS)
 *    are rounded to bfloat16 (round-to-nearest-even) before the bf16 matrix
 *    products, or carried as bf16 pairs (enum fa_precision, backward); the
 *    scale is applied in fp32 to the fp32 scores, never folded into a rounded
 *    operand. NaN or Inf in an input row propagates to the outputs that
 *    depend on it; masked scores are replaced, not multiplied, so a NaN key
 *    row does not reach the causal rows before it. Where a product spans a
 *    whole tile, a NaN also reaches outputs of the same tile through a zero
 *    factor: a NaN in query row i sets dK_j to NaN for the keys i < j <=
 *    32 * floor(i / 32) + 31 as well (64 * floor(i / 64) + 63 with
 *    FA_PRECISION_BF16 at head_dim 64, and at head_dim 128 for causal calls
 *    with n_q_heads == n_kv_heads and seqlen_k <= 1024): the dK/dV pass
 *    multiplies aligned 32-row (64-row) blocks of Q, and 0 * NaN is NaN.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad sizes, non-finite scale */
  FA_ERR_UNSUPPORTED = 2,      /* head_dim, dtype combination, causal with seqlen_q != seqlen_k */
  FA_ERR_HIP = 3               /* a HIP launch failed; fa_last_error() has the text */
};

/* Element types. */
enum fa_dtype {
  FA_DTYPE_F32 = 0,
  FA_DTYPE_BF16 = 1
};

/* How the backward passes feed the probabilities P and their gradients dS
 * to the bf16 matrix products dV = P^T dO, dK = dS^T Q, dQ = dS K.
 *  FA_PRECISION_BF16: each is rounded once to bf16 (round-to-nearest-even),
 *    the 16-bit products of the pages (CSDN FlashAttention-2 article, the
 *    FP16/BF16 matrix multiplies): relative error up to 2^-9 per element.
 *  FA_PRECISION_HILO: each is carried as a pair of bf16 values hi + lo, with
 *    hi = RNE(x) and lo = RNE(x - hi) (x - hi is exact in fp32), and enters
 *    two products, one per term: relative error up to 2^-18 per element, at
 *    the cost of one more product per gradient (7 instead of 5 per score
 *    pair, 10 instead of 7 in fa_bwd's two passes). For gradients that the
 *    bf16 rounding would move by more than the caller's tolerance (grouped
 *    heads summed over many rows, near one-hot probabilities). */
enum fa_precision {
  FA_PRECISION_BF16 = 0,
  FA_PRECISION_HILO = 1
};

/*
 * fa_fwd — exact attention forward (page "6.2 FlashAttention V2 chi tiết",
 * section 6.1; CSDN FlashAttention-2 article, "前向传播").
 *
 *   q        [B][Hq][Nq][d]  in_dtype, read only
 *   k, v     [B][Hkv][Nk][d] in_dtype, read only
 *   o        [B][Hq][Nq][d]  out_dtype, fully overwritten:
 *            O = softmax(scale * Q K^T, causal mask) V
 *   lse      [B][Hq][Nq] fp32, fully overwritten: L_i = m_i + ln(l_i), the
 *            natural-log logsumexp of the scaled (masked) scores of row i
 *            (page 6.2, sections 6.1 and 7.1)
 *   batch, n_q_heads, n_kv_heads  >= 1, n_q_heads % n_kv_heads == 0
 *   seqlen_q, seqlen_k            >= 1; causal requires seqlen_q == seqlen_k
 *   head_dim                      64 or 128
 *   scale    any finite float (0 allowed); typically 1/sqrt(head_dim)
 *   causal   0 or 1: query i attends to keys j <= i (page 6.2, section 5.1)
 *   in_dtype  FA_DTYPE_BF16 (MFMA bf16 path) or FA_DTYPE_F32 (fp32 MFMA path,
 *             for checking the tiling at fp32 precision)
 *   out_dtype FA_DTYPE_BF16 or FA_DTYPE_F32 (any combination with in_dtype)
 *   stream   hipStream_t or NULL
 * Returns FA_OK or an fa_status code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int batch, int n_q_heads, int n_kv_heads, int seqlen_q, int seqlen_k,
           int head_dim, float scale, int causal, int in_dtype, int out_dtype,
           void* stream);

/*
 * fa_bwd — exact attention backward (page "6.2 FlashAttention V2 chi tiết",
 * section 7; CSDN FlashAttention-2 article, "3.1.2 反向传播公式解析"):
 *   D = rowsum(dO o O); P = exp(scale * Q K^T - L) (masked);
 *   dV = P^T dO; dP = dO V^T; dS = P o (dP - D);
 *   dQ = scale * dS K; dK = scale * dS^T Q;
 * with dK, dV summed over the query heads of each K/V head group.
 *
 * Scheme: a pass over Q tiles forms D once per row (section 7.3) and dQ
 * (the "two-pass" alternative to atomics that section 7.2 names); then dK
 * and dV by workgroups that each own one K/V column block (section 7.2),
 * reading D. No atomics are used and every output is deterministic.
 * fa_bwd_atomic below is the single-pass variant.
 *
 *   q, dout  [B][Hq][Nq][d] in_dtype (must be FA_DTYPE_BF16), read only
 *   k, v     [B][Hkv][Nk][d] in_dtype, read only
 *   o        [B][Hq][Nq][d] o_dtype (bf16 or fp32), the forward output
 *   lse      [B][Hq][Nq] fp32, the forward logsumexp
 *   dq       [B][Hq][Nq][d] fp32, fully overwritten
 *   dk, dv   [B][Hkv][Nk][d] grad_dtype (bf16 or fp32), fully overwritten
 *   workspace  device buffer of at least fa_bwd_workspace_bytes() bytes; on
 *            return it holds D as fp32 [B][Hq][Nq]
 *   precision  FA_PRECISION_BF16 or FA_PRECISION_HILO (enum fa_precision)
 *   other arguments as in fa_fwd.
 * Returns FA_OK or an fa_status code.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, float* dq, void* dk, void* dv,
           float* workspace, int batch, int n_q_heads, int n_kv_heads,
           int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
           int in_dtype, int o_dtype, int grad_dtype, int precision,
           void* stream);

/*
 * fa_bwd_atomic — the same computation, arguments and results as fa_bwd, in
 * a single pass: the K/V-column-block workgroups also form dQ_i = dS K_j for
 * every Q block they visit and add it to dq with fp32 atomics (page 6.2,
 * section 7.2; CSDN article, "并行性 / 反向传播"); the preprocess kernel
 * zeroes dq first. Fewer matrix products than fa_bwd, but the atomic traffic
 * is (number of K/V blocks) * seqlen_q * head_dim * 4 bytes per query head,
 * and the last bits of dq depend on the order of the atomic adds. precision
 * must be FA_PRECISION_BF16 (FA_ERR_UNSUPPORTED otherwise).
 */
int fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, float* dq, void* dk,
                  void* dv, float* workspace, int batch, int n_q_heads,
                  int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim,
                  float scale, int causal, int in_dtype, int o_dtype,
                  int grad_dtype, int precision, void* stream);

/* Largest batch * n_q_heads * seqlen_q that fa_bwd_noalloc accepts. */
#define FA_BWD_NOALLOC_MAX_ROWS 4194304

/*
 * fa_bwd_noalloc — fa_bwd without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The library keeps D in a static
 * device array of FA_BWD_NOALLOC_MAX_ROWS fp32 values (16 MiB), one per
 * device, created with the library's code on that device and held until the
 * process ends; the call itself allocates nothing. Results are those of
 * fa_bwd with the same arguments (the same kernels). The caller still
 * allocates q, k, v, o, lse, dout, dq, dk, dv as for fa_bwd.
 *   batch * n_q_heads * seqlen_q > FA_BWD_NOALLOC_MAX_ROWS:
 *            FA_ERR_INVALID_ARGUMENT, before anything is enqueued.
 *   Every call on a device uses that device's one array: calls that may run
 *   at the same time on one device (different streams, other host threads)
 *   race on it and must be serialised by the caller.
 * Other arguments, ownership and errors as in fa_bwd.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, float* dq, void* dk,
                   void* dv, int batch, int n_q_heads, int n_kv_heads,
                   int seqlen_q, int seqlen_k, int head_dim, float scale,
                   int causal, int in_dtype, int o_dtype, int grad_dtype,
                   int precision, void* stream);

/*
 * fa_fwd_varlen — fa_fwd on a packed batch of sequences of different lengths
 * (the variable-length batches named on the FlashAttention-3 news page among
 * its next steps): sequence b's queries are rows [cu_seqlens_q[b],
 * cu_seqlens_q[b+1]) of the packed query arrays and its keys rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of the packed key arrays; each
 * sequence is attended on its own, exactly as fa_fwd with batch 1 would.
 *
 *   q, o     [Hq][total_q][d] (o in out_dtype), packed by head then row
 *   k, v     [Hkv][total_k][d]
 *   lse      [Hq][total_q] fp32
 *   cu_seqlens_q, cu_seqlens_k  device int32 arrays of batch + 1
 *            non-decreasing offsets, cu[0] = 0, cu[batch] = total; read
 *            only. Offsets are clamped to [0, total] and lengths to
 *            max_seqlen, so malformed arrays give wrong rows but no access
 *            outside the packed arrays.
 *   max_seqlen_q, max_seqlen_k  at least every sequence's length (0 allowed)
 *   in_dtype must be FA_DTYPE_BF16.
 *   causal: token i of a sequence sees that sequence's keys 0..i; requires
 *            the same sequences for queries and keys (cu_seqlens_q ==
 *            cu_seqlens_k as pointers, equal max_seqlen and total), else
 *            FA_ERR_UNSUPPORTED.
 * A sequence with queries but no keys gets O = 0 and L = -inf. Other
 * arguments, ownership and errors as in fa_fwd.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                  int total_k, int n_q_heads, int n_kv_heads, int head_dim,
                  float scale, int causal, int in_dtype, int out_dtype,
                  void* stream);

/*
 * fa_bwd_varlen — fa_bwd (two passes, no atomics) on a packed batch laid out
 * as in fa_fwd_varlen: dq [Hq][total_q][d] fp32; dk, dv [Hkv][total_k][d]
 * grad_dtype; o, dout [Hq][total_q][d]; lse [Hq][total_q]; workspace of at
 * least fa_bwd_workspace_bytes(1, n_q_heads, total_q) bytes, holding D as
 * fp32 [Hq][total_q] on return. dq, dk and dv are fully overwritten (keys of
 * a sequence without queries get dK = dV = 0; queries without keys dQ = 0).
 * precision as in fa_bwd.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, float* dq, void* dk,
                  void* dv, float* workspace, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int batch, int max_seqlen_q,
                  int max_seqlen_k, int total_q, int total_k, int n_q_heads,
                  int n_kv_heads, int head_dim, float scale, int causal,
                  int in_dtype, int o_dtype, int grad_dtype, int precision,
                  void* stream);

/*
 * fa_quantize_fp8 — the FP8 quantization with incoherent processing of the
 * FlashAttention-3 news page ("Độ chính xác thấp FP8 và incoherent
 * processing"): each row x of a [B][H][N][d] bf16 tensor becomes
 *   y = FWHT(x o s) / sqrt(d)       (s = signs, +-1 per channel; FWHT the
 *                                    unnormalised Walsh-Hadamard transform)
 * or y = x when signs is NULL; then every block of 64 rows (the last one may
 * be shorter) of one (batch, head) gets the scale 2^e, the smallest power of
 * two with max|y| <= 448 * 2^e and e >= -126 (e = 0 for an all-zero block;
 * inputs must be finite), and its elements are stored as OCP FP8 E4M3
 * codes of y / 2^e, rounded to nearest, ties to even. Applying the same
 * signs to Q and K leaves Q K^T unchanged (the transform is orthogonal) while
 * spreading outlier channels over all channels.
 *   x            device, bf16 [B][H][N][d] (in_dtype must be FA_DTYPE_BF16),
 *                16-byte aligned
 *   codes        device, uint8 [B][H][N][d], 16-byte aligned, overwritten
 *   block_scales device, fp32 [B][H][ceil(N/64)] (fa_fp8_scales_count
 *                entries), overwritten with the powers of two 2^e
 *   signs        device int8 [d] of +1 / -1, or NULL for no transform
 *   head_dim     64 or 128
 * The transform runs in fp32 as a fixed sequence of butterflies (a + b,
 * a - b) over stages h = 1, 2, 4, ..., d/2, then one multiply by
 * fp32(1/sqrt d), so the codes are reproducible bit for bit.
 */
int fa_quantize_fp8(const void* x, void* codes, float* block_scales,
                    const signed char* signs, int batch, int n_heads,
                    int seqlen, int head_dim, int in_dtype, void* stream);

/* Number of block scales fa_quantize_fp8 writes: batch * n_heads *
 * ceil(seqlen / 64) (0 for non-positive arguments). */
size_t fa_fp8_scales_count(int batch, int n_heads, int seqlen);

/*
 * fa_quantize_vt_fp8 — V for the FP8 P V product (fa_fwd_fp8_pv): per 64-key
 * block of one head, the power-of-two scale 2^e with max|v| <= 448 * 2^e
 * (as fa_quantize_fp8, no transform) and the e4m3 codes of v / 2^e (round to
 * nearest even), written transposed: block j of head h occupies
 * vt_codes[((h * ceil(N/64)) + j) * d * 64 ..] as d rows of 64 codes, row c
 * holding channel c of the block's keys in the order the forward's product
 * consumes them: position 32 g + s (g = 0, 1; s < 32) holds key
 * 32 (s / 16) + 8 ((s % 16) / 4) + 4 g + s % 4 of the block; keys past N get
 * code 0. (FlashAttention-3 news page, "Độ chính xác thấp FP8 và incoherent
 * processing", and its mention of the FP8 transpose: the transpose is done
 * here, in the pass that rewrites V anyway.)
 *   v            device, bf16 [B][H][N][d], 16-byte aligned
 *   vt_codes     device, uint8, fa_fp8_vt_bytes(B, H, N, d) bytes, 16-byte aligned
 *   block_scales device, fp32 [B][H][ceil(N/64)], 4-byte aligned
 * head_dim 64 or 128; in_dtype FA_DTYPE_BF16. Asynchronous on stream.
 */
int fa_quantize_vt_fp8(const void* v, void* vt_codes, float* block_scales,
                       int batch, int n_heads, int seqlen, int head_dim,
                       int in_dtype, void* stream);

/* Bytes fa_quantize_vt_fp8 writes: batch * n_heads * ceil(seqlen / 64) * 64
 * * head_dim (0 for non-positive arguments). */
size_t fa_fp8_vt_bytes(int batch, int n_heads, int seqlen, int head_dim);

/*
 * fa_fwd_fp8_pv — fa_fwd_fp8 with the second product in FP8 as well: P is
 * rounded to e4m3 at the fixed scale 2^8 against the running row maximum of
 * the key tiles seen so far (the largest probability is exactly 1), V comes
 * as the transposed codes and block scales of fa_quantize_vt_fp8, and
 * O^T += V^T P^T runs on the FP8 matrix cores; the row sum l is accumulated
 * in fp32 over the unrounded probabilities, so L is that of fa_fwd_fp8.
 *   q_codes, q_scales, k_codes, k_scales as in fa_fwd_fp8 (d = 64 or 128);
 *   vt_codes, v_scales as written by fa_quantize_vt_fp8 for V [B][Hkv][Nk][d];
 *   o, lse, scale, causal, out_dtype as in fa_fwd.
 */
int fa_fwd_fp8_pv(const void* q_codes, const float* q_scales, const void* k_codes,
                  const float* k_scales, const void* vt_codes, const float* v_scales,
                  void* o, float* lse, int batch, int n_q_heads, int n_kv_heads,
                  int seqlen_q, int seqlen_k, int head_dim, float scale, int causal,
                  int out_dtype, void* stream);

/*
 * fa_fwd_fp8_quantize_q — fa_fwd_fp8 (v_scales NULL) or fa_fwd_fp8_pv
 * (v_scales given) with Q taken in bf16 and quantized inside the forward,
 * exactly as fa_quantize_fp8 would with the same signs (the same butterflies
 * in the same order, the same 64-row block scales, the same codes), so the
 * outputs equal those of fa_quantize_fp8 followed by fa_fwd_fp8 /
 * fa_fwd_fp8_pv bit for bit, without the separate pass over Q (FlashAttention-3
 * news page, "Độ chính xác thấp FP8 và incoherent processing": the transform
 * can be fused with the memory-bound work around it). Q's codes and scales
 * are not written out.
 *   q        device, bf16 [B][Hq][Nq][d], 16-byte aligned; finite
 *   q_signs  device int8 [d] of +1 / -1 (the signs K was quantized with), or
 *            NULL for no transform
 *   k_codes, k_scales as in fa_fwd_fp8
 *   v        bf16 [B][Hkv][Nk][d] if v_scales is NULL, else the transposed
 *            codes of fa_quantize_vt_fp8 with their block scales v_scales
 *   o, lse, scale, causal, out_dtype as in fa_fwd; head_dim 64 or 128.
 * Errors as fa_fwd_fp8; k_scales NULL or a misaligned scale array is
 * FA_ERR_INVALID_ARGUMENT. Asynchronous on stream.
 */
int fa_fwd_fp8_quantize_q(const void* q, const signed char* q_signs,
                          const void* k_codes, const float* k_scales,
                          const void* v, const float* v_scales, void* o,
                          float* lse, int batch, int n_q_heads, int n_kv_heads,
                          int seqlen_q, int seqlen_k, int head_dim, float scale,
                          int causal, int out_dtype, void* stream);

/*
 * fa_fwd_fp8 — fa_fwd with the scores formed in FP8: q_codes / k_codes and
 * q_scales / k_scales as written by fa_quantize_fp8 (with the same signs for
 * Q and K), S = scale * (Q_codes 2^e_q)(K_codes 2^e_k)^T by FP8 matrix cores
 * (fp32 accumulate, one block scale pair per 64 x 64 score tile), then the
 * online softmax and O = P V exactly as fa_fwd (P rounded to bf16, V bf16).
 *   q_codes [B][Hq][Nq][d], k_codes [B][Hkv][Nk][d] uint8, 16-byte aligned
 *   q_scales [B][Hq][ceil(Nq/64)], k_scales [B][Hkv][ceil(Nk/64)] fp32
 *   v [B][Hkv][Nk][d] bf16; o, lse, scale, causal, out_dtype as in fa_fwd.
 * head_dim (d) 64 or 128 (else FA_ERR_UNSUPPORTED).
 */
int fa_fwd_fp8(const void* q_codes, const float* q_scales, const void* k_codes,
               const float* k_scales, const void* v, void* o, float* lse,
               int batch, int n_q_heads, int n_kv_heads, int seqlen_q,
               int seqlen_k, int head_dim, float scale, int causal,
               int out_dtype, void* stream);

/*
 * fa_fwd_persistent — fa_fwd (bf16 q, k, v) on a persistent grid fed by a
 * work queue: the causal scheduler of the FlashAttention-3 news page
 * (on persistent kernels). As many workgroups as the device keeps resident
 * pull (batch, query head, Q tile) items, heaviest causal tile first, from
 * per-XCD queues, and take the lightest remaining items of the other queues
 * when their own is empty. Results are bit-identical to fa_fwd's 4-wavefront
 * kernel for the same inputs (the same per-item arithmetic).
 *   sched  device int array of fa_fwd_persistent_sched_bytes() bytes,
 *          4-byte aligned, all zero before the first call; every call leaves
 *          it zero when it completes. Calls that may run at the same time
 *          (different streams) need separate arrays.
 *   other arguments as in fa_fwd; in_dtype must be FA_DTYPE_BF16.
 */
int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o,
                      float* lse, int* sched, int batch, int n_q_heads,
                      int n_kv_heads, int seqlen_q, int seqlen_k, int head_dim,
                      float scale, int causal, int in_dtype, int out_dtype,
                      void* stream);

/* Bytes of the work-queue counter array fa_fwd_persistent needs (36). */
size_t fa_fwd_persistent_sched_bytes(void);

/* Bytes of device workspace fa_bwd and fa_bwd_atomic need: 4 * batch * n_q_heads * seqlen_q
 * (the fp32 vector D, page 6.2 section 7.3). Returns 0 for non-positive
 * arguments. */
size_t fa_bwd_workspace_bytes(int batch, int n_q_heads, int seqlen_q);

/* Static text for a status code (never NULL). */
const char* fa_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* fa_last_error(void);

/* Library ABI version, currently 2 (2 added the precision argument of the
 * backward entry points). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
