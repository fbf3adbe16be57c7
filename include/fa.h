/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library with a per-token
 * int8 KV cache.
 *
 * The operations and where they are defined:
 *   fa_compress_kv  -- per-token int8 quantization with one fp32 scale per token
 *                      (fkl.flash_attention PR, "FA-2 forward with fused epilogue +
 *                      compressed int8 KV cache", Summary: compress_kv()).
 *   fa_forward      -- exact softmax(Q K^T * scale) V as a FlashAttention-2 style
 *                      forward with causal / ragged / GQA / sliding-window masks, the
 *                      Mul/Add epilogue chain and int8 K/V dequantized inside q.k and
 *                      p.v (fkl PR, Summary: flash_attention(), epilogue=[...], layout
 *                      and precision bullet; SKaiNET PR #419, Summary: GQA groups and
 *                      sliding-window layers).
 *   fa_append_kv    -- the decode-time cache write: new K/V tokens quantized by the
 *                      same rule into the int8 cache at device-held positions (fkl PR,
 *                      Summary: the compressed cache holds K/V for long-context decode).
 *   fa_merge_lse    -- exact attention over a union of key chunks from the chunks'
 *                      normalised outputs and log-sum-exps, the state a split or ring
 *                      prefill exchanges (kernbench2 ADR-0060 commit: partial (m, l, O)
 *                      states reduced into one).
 *   fa_tq_codebook, fa_tq_encode, fa_tq_decode
 *                   -- the TurboQuant 2-4-bit KV codec: randomized Hadamard rotation,
 *                      L2 normalisation, Lloyd-Max codebook of the Beta(d/2, d/2)
 *                      coordinate law, bit-packing (Foundry attention/ README, section
 *                      "TurboQuant KV Cache Compression").
 *   fa_decode       -- one query row per head against an int8 cache, split over the
 *                      keys with a log-sum-exp merge of the partial (m, l, O) states
 *                      (fkl PR, Verification: the decode check; kernbench2 ADR-0060
 *                      commit: split decode with a reduce of running (m, l, O)).
 *
 * Conventions shared by every entry point
 *   Layout      (batch*heads, seq, head_dim), row-major and contiguous; head_dim is a
 *               multiple of 32 and at most FA_MAX_HEAD_DIM (fkl PR, Summary).
 *   Pointers    device pointers unless stated; 16-byte aligned.  The caller allocates
 *               and owns every buffer; the library allocates no device memory and keeps
 *               no pointer after a call returns.
 *   Streams     `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *               asynchronously; nothing synchronises the host.
 *   Errors      every argument is checked on the host before anything is enqueued.  On
 *               error a negative fa_status is returned, nothing is enqueued or written,
 *               and fa_last_error() gives the reason on the calling thread.
 *               No exception or abort crosses the ABI.
 *   Precision   accumulation is fp32 everywhere (fkl PR, Summary).
 *   GQA         G = bh_q / bh_kv must be an integer; query head h reads KV head h / G.
 *   Causal      bottom-right aligned: query row i sees key j iff j <= i + (s_k - s_q).
 *   Window      W > 0 keeps keys with i' - W < j <= i' (W counts the diagonal);
 *               only together with causal.  W >= s_k is the same as plain causal.
 *   Empty rows  a query row with no visible key returns 0 (and LSE = -inf).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,      /* null/misaligned pointer, bad size, inconsistent arguments */
  FA_ERR_UNSUPPORTED = -2,  /* head_dim, dtype combination or epilogue length not supported */
  FA_ERR_WORKSPACE = -3,    /* decode workspace missing or too small */
  FA_ERR_HIP = -4           /* the HIP runtime reported an error (text in fa_last_error) */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_I8 = 2 } fa_dtype;

typedef enum { FA_EPI_MUL = 1, FA_EPI_ADD = 2, FA_EPI_BIAS = 3, FA_EPI_RELU = 4 } fa_epi_kind;

/* One epilogue post-op, applied in fp32 to the normalised attention output, in list order,
 * before the cast to the output dtype (fkl PR, Summary: epilogue=[Mul(2.0), Add(0.5)] -- any
 * compute ops chained on the output; kernbench2 commit page, the commit that gives
 * tl.composite() an ordered epilogue list of bias, relu and scale ops).  Each op is one separately rounded IEEE fp32 operation:
 *   FA_EPI_MUL   x * value            FA_EPI_ADD   x + value
 *   FA_EPI_BIAS  x + vec[c], c the head-dim index of the element; vec is a device fp32 array
 *                of head_dim values (4-byte aligned), required for this kind and NULL otherwise
 *   FA_EPI_RELU  x > 0 ? x : +0 (value unused)
 * Every op carries a scope (kernbench2 commit page, the same commit: each tl.composite() op is
 * flagged output_tile, the default, k_tile, run on every K tile right after its GEMM, or kernel):
 *   FA_SCOPE_OUTPUT_TILE  (0, so a zero-initialised op keeps the behaviour above) the normalised
 *                         output row, as described above.
 *   FA_SCOPE_K_TILE       every raw score x = q.k_j of a key tile (K dequantized), before the
 *                         mask and the softmax scale: the softmax then sees scale * f(x).  For
 *                         FA_EPI_BIAS, vec[j] is added, j the key position in [0, s_k): vec is a
 *                         device fp32 array of s_k values shared by all heads.  Accepted by
 *                         fa_forward, fa_decode, fa_decode_noalloc and fa_tq_attention_decode;
 *                         fa_merge_lse, which forms no scores, returns FA_ERR_UNSUPPORTED.
 *   FA_SCOPE_KERNEL       FA_ERR_UNSUPPORTED: no step of attention runs once per kernel.
 * The ops of each scope run in their list order; both scopes together hold at most
 * FA_MAX_EPILOGUE ops.  Values, vectors and the list itself are kernel arguments: changing them
 * never selects another kernel (fkl PR, Verification: epilogue values change without
 * recompile); only whether any K-tile op is present does (an instantiation whose
 * fa_last_kernel name ends in "_sops"). */
typedef enum { FA_SCOPE_OUTPUT_TILE = 0, FA_SCOPE_K_TILE = 1, FA_SCOPE_KERNEL = 2 } fa_epi_scope;

typedef struct {
  int32_t kind;        /* fa_epi_kind */
  float value;         /* FA_EPI_MUL / FA_EPI_ADD */
  const float* vec;    /* FA_EPI_BIAS: device [head_dim] (output scope) or [s_k] (K-tile scope);
                          NULL for the other kinds */
  int32_t scope;       /* fa_epi_scope */
} fa_epilogue_op;

#define FA_MAX_EPILOGUE 8
#define FA_MAX_HEAD_DIM 256

/*
 * fa_compress_kv -- quantize n_tokens rows of head_dim values to int8 codes + fp32 scales.
 *   x          device, [n_tokens, head_dim], FA_F32 or FA_BF16 (x_dtype).
 *   q_out      device, [n_tokens, head_dim] int8.
 *   scale_out  device, [n_tokens] fp32.
 * Per token: a = max|x|, s = a / 127 (IEEE fp32 division), q = rint(x / s) (IEEE fp32
 * quotient, ties to even) clamped to [-127, 127]; an all-zero token gives s = 0, q = 0.
 * Outputs may not alias x.  n_tokens == 0 is a no-op that returns FA_OK.
 */
int fa_compress_kv(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t head_dim,
                   int8_t* q_out, float* scale_out, void* stream);

/*
 * fa_append_kv -- quantize n_new new tokens per KV head of K and of V into an int8 cache.
 *   k_new, v_new     device, [bh_kv, n_new, head_dim], x_dtype FA_F32 or FA_BF16.
 *   pos              device int32 [bh_kv]: token j of KV head b goes to cache row pos[b] + j.
 *                    Read on the device, so the call can be replayed (for instance from a
 *                    captured graph) while the caller advances the positions; different heads
 *                    (sequences) may sit at different lengths.
 *   k_cache, v_cache device int8 [bh_kv, capacity, head_dim]; k_scale, v_scale device fp32
 *                    [bh_kv, capacity].  Rows outside [0, capacity) are skipped, never written.
 * Codes and scales are bit-identical to fa_compress_kv of the same rows (fkl PR, Summary:
 * compress_kv(), one fp32 scale per token).  Inputs may not alias the caches.
 * n_new == 0 is a no-op that returns FA_OK.
 */
int fa_append_kv(const void* k_new, const void* v_new, int32_t x_dtype, int32_t bh_kv, int32_t n_new,
                 int32_t head_dim, const int32_t* pos, int32_t capacity, int8_t* k_cache, int8_t* v_cache,
                 float* k_scale, float* v_scale, void* stream);

/*
 * fa_append_kv_rope -- fa_append_kv with the new K rows first rotated by rotate-half RoPE at their
 * cache position (FlashRT QKV Cache RoPE, Kernels list: the decode K write applies rotate-half RoPE
 * with half-width cos/sin vectors and selects the slot from a device position).
 *   rope_cos, rope_sin  device fp32 [capacity, head_dim / 2], 16-byte aligned: row p holds the
 *                       cos / sin of cache position p.  Both NULL: no rotation (fa_append_kv).
 * For channel i < head_dim / 2 and the K row x written at position p:
 *   x'_i = x_i cos[p][i] - x_{i+d/2} sin[p][i],  x'_{i+d/2} = x_{i+d/2} cos[p][i] + x_i sin[p][i],
 * each product and the sum a separately rounded fp32 operation; x' is then quantized exactly as
 * fa_compress_kv quantizes a row.  V rows are written unrotated.  Other arguments, skipping and
 * errors as for fa_append_kv.
 */
int fa_append_kv_rope(const void* k_new, const void* v_new, int32_t x_dtype, int32_t bh_kv, int32_t n_new,
                      int32_t head_dim, const int32_t* pos, int32_t capacity, const float* rope_cos,
                      const float* rope_sin, int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                      void* stream);

/*
 * fa_forward -- attention forward for bh_q query heads over bh_kv KV heads.
 *   q        device, [bh_q, s_q, head_dim], q_dtype FA_F32 or FA_BF16.
 *   k, v     device, [bh_kv, s_k, head_dim], kv_dtype FA_F32, FA_BF16 or FA_I8.
 *   k_scale, v_scale  device, [bh_kv, s_k] fp32 per-token scales; required iff kv_dtype is
 *            FA_I8 (values are then q * s, dequantized in registers), NULL otherwise.
 *   out      device, [bh_q, s_q, head_dim], out_dtype FA_F32 or FA_BF16 (RNE cast).
 *   lse_out  device or NULL, [bh_q, s_q] fp32 natural-log log-sum-exp of the scaled scores.
 *   softmax_scale  <= 0 selects 1/sqrt(head_dim).
 *   causal, window  see the conventions above; window > 0 requires causal.
 *   epi, n_epi      host array of n_epi (<= FA_MAX_EPILOGUE) post-ops, may be NULL if 0.
 * Supported (q_dtype, kv_dtype): (F32, F32), (F32, I8), (BF16, BF16), (BF16, I8).
 * s_q == 0 is a no-op; s_k == 0 with s_q > 0 writes zeros (every row is empty).
 */
int fa_forward(const void* q, int32_t q_dtype,
               const void* k, const void* v, int32_t kv_dtype,
               const float* k_scale, const float* v_scale,
               void* out, int32_t out_dtype, float* lse_out,
               int32_t bh_q, int32_t bh_kv, int32_t s_q, int32_t s_k, int32_t head_dim,
               float softmax_scale, int32_t causal, int32_t window,
               const fa_epilogue_op* epi, int32_t n_epi, void* stream);

/*
 * fa_merge_lse -- merge n_parts attention results for the same `rows` query rows, each over
 * its own disjoint set of keys, into the result over all of them.
 *   o_parts    device fp32 [n_parts, rows, head_dim]: each part's normalised output, as
 *              fa_forward writes it with out_dtype FA_F32 and no epilogue.
 *   lse_parts  device fp32 [n_parts, rows]: each part's log-sum-exp (fa_forward's lse_out;
 *              -inf for a row with no visible key in that part).
 *   out        device [rows, head_dim], out_dtype FA_F32 or FA_BF16 (RNE cast).
 *   lse_out    device or NULL, [rows] fp32.
 *   epi, n_epi the Mul/Add epilogue, applied once to the merged row before the cast.
 * LSE = log sum_p exp(LSE_p); out = sum_p exp(LSE_p - LSE) O_p, computed against the largest
 * LSE_p; a row with every LSE_p = -inf gives 0 and -inf.  With the keys split into chunks
 * aligned with chunks of the queries, each (query chunk, key chunk) part is either fully
 * visible, a causal diagonal block, or empty, so a causal prefill splits into fa_forward calls
 * and one merge (the exchange of a ring / context-parallel prefill).
 * rows == 0 is a no-op.  out may not alias the inputs.
 */
int fa_merge_lse(const float* o_parts, const float* lse_parts, int32_t n_parts, int64_t rows, int32_t head_dim,
                 void* out, int32_t out_dtype, float* lse_out, const fa_epilogue_op* epi, int32_t n_epi,
                 void* stream);

/*
 * fa_tq_codebook -- the 2^bits Lloyd-Max centroids (ascending, written to the host array
 * `centroids`) of u = 2B - 1 with B ~ Beta(head_dim/2, head_dim/2), the coordinate law the
 * TurboQuant page quantizes against (Foundry attention/ README, TurboQuant section).  Computed
 * on the host (Lloyd-Max iterations, Gauss-Legendre quadrature), about 0.1 s; callers keep it.
 * head_dim in {32, 64, 128, 256}, bits in {2, 3, 4}.
 */
int fa_tq_codebook(int32_t head_dim, int32_t bits, float* centroids);

/*
 * fa_tq_encode -- TurboQuant codes of n_tokens vectors.
 *   x          device [n_tokens, head_dim], FA_F32 or FA_BF16.
 *   signs      device int8 [head_dim], each +1 or -1: the random diagonal of the rotation.
 *   codebook   host fp32 [2^bits], strictly increasing and antisymmetric (c[k] == -c[2^bits-1-k],
 *              as the codebook of a symmetric law is; fa_tq_codebook's output), else FA_ERR_INVALID.
 *   codes_out  device uint8 [n_tokens, head_dim * bits / 8]; channel i's code at bit
 *              (i bits) mod 8 of byte (i bits) / 8.
 *   norms_out  device fp32 [n_tokens]: ||x||_2.
 * y = H (signs * x) (Sylvester Hadamard), u = y / ||y||, code_i = the number of midpoints
 * between consecutive centroids that are <= u_i.  Decisions are taken in fp32; at 4 bits they go
 * through a table of float-bit buckets when the codebook fits it (fa_last_kernel() "tq_encode",
 * as for fa_tq_codebook's codebooks) and through a search otherwise ("tq_encode_search"), with
 * the same result.
 * n_tokens == 0 is a no-op.
 */
int fa_tq_encode(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t head_dim, int32_t bits,
                 const int8_t* signs, const float* codebook, uint8_t* codes_out, float* norms_out,
                 void* stream);

/*
 * fa_tq_decode -- x_hat = signs * H (norm * codebook[code]) / sqrt(head_dim), written as out_dtype
 * (FA_F32 or FA_BF16) to device out [n_tokens, head_dim].  Arguments as for fa_tq_encode, except
 * that any strictly increasing codebook is accepted.
 */
int fa_tq_decode(const uint8_t* codes, const float* norms, int64_t n_tokens, int32_t head_dim, int32_t bits,
                 const int8_t* signs, const float* codebook, void* out, int32_t out_dtype, void* stream);

/*
 * fa_tq_attention_decode -- one decode step (as fa_decode) over a KV cache held as TurboQuant
 * codes, read directly: the codes are turned into matrix-core operands in registers and the
 * decoded cache is never written to memory (Foundry attention/ README, section "TurboQuant KV
 * Cache Compression": K and V stored as rotated, normalised Lloyd-Max codes; fkl PR, Summary:
 * the compressed cache is dequantized inside q.k and p.v).  The result is attention over
 *   K^_j = k_signs * H (k_norms_j k_codebook[code_j]) / sqrt(d), V^_j likewise,
 * the vectors fa_tq_decode would produce: scores use q' = H (k_signs * q) against the codebook,
 * P.V is accumulated in the rotated domain and rotated back once per head.
 *   q          device [bh_q, 1, head_dim], FA_BF16 or FA_F32.
 *   k_codes    device uint8 [bh_kv, s_k, head_dim k_bits / 8] as fa_tq_encode writes them;
 *              k_norms device fp32 [bh_kv, s_k]; k_signs device int8 [head_dim]; k_codebook host
 *              fp32 [2^k_bits], strictly increasing; likewise for V.
 *   k_bits, v_bits  2, 3 or 4 (3-bit codes straddle bytes in the packed stream; the kernel
 *                   widens each 24-bit run of 8 codes to 4-bit fields in registers).
 *                   head_dim 64 or 128.
 *   out, lse_out, softmax_scale, window, num_splits, epi, workspace: as for fa_decode, with
 *              fa_tq_attention_num_splits / fa_tq_attention_workspace_bytes for the sizes.
 * The codebooks enter as three 7-bit digits each (2^-22 of their largest entry); all other
 * arithmetic is exact in integers or fp32.
 */
int fa_tq_attention_decode(const void* q, int32_t q_dtype,
                           const uint8_t* k_codes, const float* k_norms, const int8_t* k_signs, int32_t k_bits,
                           const float* k_codebook,
                           const uint8_t* v_codes, const float* v_norms, const int8_t* v_signs, int32_t v_bits,
                           const float* v_codebook,
                           void* out, int32_t out_dtype, float* lse_out,
                           int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim,
                           float softmax_scale, int32_t window, int32_t num_splits,
                           const fa_epilogue_op* epi, int32_t n_epi,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Split count and workspace bytes of fa_tq_attention_decode (num_splits 0 = automatic). */
int32_t fa_tq_attention_num_splits(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim);
size_t fa_tq_attention_workspace_bytes(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim,
                                       int32_t num_splits);

/*
 * fa_decode_num_splits -- the split count fa_decode uses when num_splits == 0.
 */
int32_t fa_decode_num_splits(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim);

/*
 * fa_decode_workspace_bytes -- device workspace fa_decode needs for these sizes
 * (num_splits == 0 means the automatic count).  The workspace holds one partial
 * (m, l, O[head_dim]) per (query head, split), fp32.
 */
size_t fa_decode_workspace_bytes(int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim,
                                 int32_t num_splits);

/*
 * fa_decode -- one decode step: each of the bh_q query heads has one row that sees the whole
 * int8 cache of its KV head (or its last `window` keys), computed as a split-KV pass that
 * writes partial (m, l, O) states to `workspace` followed by a log-sum-exp merge pass.
 *   q        device, [bh_q, 1, head_dim], FA_BF16 or FA_F32.
 *   k, v     device int8 codes [bh_kv, s_k, head_dim]; k_scale, v_scale device fp32 [bh_kv, s_k].
 *   out      device, [bh_q, 1, head_dim], FA_F32 or FA_BF16.
 *   lse_out  device or NULL, [bh_q] fp32.
 *   num_splits  0 = automatic; otherwise 1..4096.
 *   workspace   device, at least fa_decode_workspace_bytes(...) bytes, 16-byte aligned.
 * The result may differ with num_splits only by fp32 rounding.
 */
int fa_decode(const void* q, int32_t q_dtype,
              const int8_t* k, const int8_t* v, const float* k_scale, const float* v_scale,
              void* out, int32_t out_dtype, float* lse_out,
              int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim,
              float softmax_scale, int32_t window, int32_t num_splits,
              const fa_epilogue_op* epi, int32_t n_epi,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc -- fa_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as fa_decode (bit for bit
 * at the same num_splits), except that the partial (m, l, O) states go to a fixed device array
 * inside the library, fa_decode_noalloc_max_bytes() bytes (4 MiB) per GPU, held from the first
 * call on that GPU until the process ends.  The states need bh_q * splits * (head_dim + 2) * 4
 * bytes; a call needing more returns FA_ERR_WORKSPACE and enqueues nothing.  `stream` must belong
 * to the current device (FA_ERR_INVALID otherwise).  Every call on one GPU shares that GPU's
 * array: calls whose kernels may overlap (concurrent streams on one GPU) race and must be
 * serialised by the caller.  The caller still provides q, the cache, out and lse_out.
 */
int fa_decode_noalloc(const void* q, int32_t q_dtype,
                      const int8_t* k, const int8_t* v, const float* k_scale, const float* v_scale,
                      void* out, int32_t out_dtype, float* lse_out,
                      int32_t bh_q, int32_t bh_kv, int32_t s_k, int32_t head_dim,
                      float softmax_scale, int32_t window, int32_t num_splits,
                      const fa_epilogue_op* epi, int32_t n_epi, void* stream);

/* Size in bytes of the fixed scratch array fa_decode_noalloc uses on each GPU. */
size_t fa_decode_noalloc_max_bytes(void);

/* Text for the last non-OK return on the calling thread ("" if none).  Valid until the
 * next library call on this thread. */
const char* fa_last_error(void);

/* Name of the kernel instantiation the last successful launch on this thread used.  It
 * depends only on dtypes, head_dim and the mask family, never on epilogue values or length. */
const char* fa_last_kernel(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
