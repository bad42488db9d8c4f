/*
 * xk.h -- C ABI of the MI355X (gfx950) DeepSeek-V4 DSA indexer hot path.
 *
 * The operations, each asynchronous on the caller's HIP stream:
 *   xk_indexer_logits        weighted-ReLU MQA score over all keys (bf16 or OCP fp8)
 *   xk_indexer_logits_paged  the same score with keys in a paged mxfp4 / fp8 cache
 *   xk_indexer_topk          deterministic per-query top-k of those scores
 *   xk_indexer_logits_topk   both at once, without the score matrix for prefill shapes
 *   xk_indexer_logits_topk_noalloc  the same with built-in scratch, for callers that cannot allocate
 *   xk_mxfp4_paged_gather    mxfp4 paged KV rows of the selected keys, decoded to bf16
 *   xk_sparse_attention_mxfp4  attention of each query over its selected rows (the consumer)
 * and the producers of their quantized inputs:
 *   xk_quant_fp8_rows        per-row OCP fp8 quantizer (q per token and head, k per token)
 *   xk_mxfp4_cache_write     rows into the paged mxfp4 cache
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) unless
 *     stated otherwise; every buffer is dense row-major with the shape given.
 *     The caller owns all memory; the library allocates nothing and keeps no
 *     state between calls (apart from a per-device "is this gfx950" cache
 *     and the built-in scratch of xk_indexer_logits_topk_noalloc), so calls
 *     on different streams or threads are independent (except that one).
 *   - `stream` is the caller's hipStream_t (NULL = the null stream). A
 *     call only enqueues kernels: outputs are valid once the stream reaches
 *     them, and inputs must stay untouched until then. Nothing synchronises.
 *   - Element offsets are computed in 64 bits (paged-MQA kernels on the pages
 *     needed 64-bit offsets once a KV buffer passed 4 GiB).
 *   - Errors: every argument is checked on the host BEFORE any HIP call; a
 *     bad argument returns XK_ERR_INVALID_ARGUMENT, a shape or device outside
 *     what the kernels implement returns XK_ERR_UNSUPPORTED, and a failed
 *     launch returns XK_ERR_HIP. On error nothing is enqueued (except
 *     XK_ERR_HIP, where the launch was attempted). xk_last_error() gives a
 *     thread-local one-line reason. No call aborts the process.
 *   - Preconditions NOT checked on the device (violating them is undefined):
 *     buffers do not alias, scales are finite and > 0, scores are not NaN,
 *     sel_pos entries >= 0 index a token the sequence has, and the block-table
 *     entries they reach lie in [0, NB).
 */
#ifndef XK_H_
#define XK_H_

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XK_OK = 0,
  XK_ERR_INVALID_ARGUMENT = 1,
  XK_ERR_UNSUPPORTED = 2,
  XK_ERR_HIP = 3
} xk_status;

typedef enum {
  XK_BF16 = 0,          /* q, k are bfloat16; no scales                        */
  XK_FP8_E4M3_OCP = 1   /* q, k are OCP e4m3fn bytes with fp32 dequant scales  */
} xk_qk_dtype;

/*
 * Indexer logits.
 *
 * Defines (page "xkernels #27 -- [AMD/MI300A] DeepSeek-V4 DSA indexer +
 * attention", comment announcing dsa_indexer_logits):
 *   logits[b,t,j] = sum_{h<H} w[b,t,h] * relu( q[b,t,h,:] . k[b,j,:] )
 * for j <= limit[b,t], and exactly -inf for limit[b,t] < j < K; one shared
 * (MQA) key per position, per-head weights, an optional causal limit,
 * fp32 logits out. With XK_FP8_E4M3_OCP the operands are the dequantized
 * values q = e4m3(q8[b,t,h,:]) * q_scale[b,t,h] and
 * k = e4m3(k8[b,j,:]) * k_scale[b,j] (the fp8 packing of the upstream kernel
 * is an encoding of the same math). No other constant enters the score.
 *
 *   q        [B,T,H,D]  bf16, or e4m3 bytes          (16-byte aligned)
 *   q_scale  [B,T,H]    fp32, fp8 only; NULL for bf16
 *   k        [B,K,D]    bf16, or e4m3 bytes          (16-byte aligned)
 *   k_scale  [B,K]      fp32, fp8 only; NULL for bf16
 *   w        [B,T,H]    fp32 head weights
 *   limit    [B,T]      int32 inclusive last valid key of each query, or NULL
 *                       (every key valid); values < 0 give an all -inf row,
 *                       values >= K are clamped to K-1
 *   logits   [B,T,K]    fp32 output; every element is written
 *   B, T, K >= 1; H must be 64 and D 128 (the DeepSeek-V4 indexer:
 *   index_n_heads 64, index_head_dim 128), B*T <= 2^30 and B*T*K <= 2^38
 *   (1 TB of logits), else XK_ERR_UNSUPPORTED.
 * Dot products accumulate in fp32 (MFMA). bf16: the ReLU, weights and head
 * sum run in fp32, so results match a float64 evaluation to ~1e-6 of
 * max|logit|. fp8: each head's ReLU'd score and weight are rounded to f16
 * before the fp32 head sum (relative error ~2^-10 per term, well inside
 * the e4m3 inputs' own 2^-4), so results match to ~1e-3 of max|logit|.
 */
xk_status xk_indexer_logits(const void* q, const float* q_scale,
                            const void* k, const float* k_scale,
                            const float* w, const int32_t* limit, float* logits,
                            int B, int T, int K, int H, int D,
                            xk_qk_dtype dtype, hipStream_t stream);

typedef enum {
  XK_KCACHE_MXFP4 = 0,        /* k_cache [NB,bs,D/2] E2M1 nibbles, k_scale [NB,bs,D/32] E8M0 */
  XK_KCACHE_FP8_E4M3_OCP = 1  /* k_cache [NB,bs,D] e4m3 bytes, k_scale [NB,bs] fp32          */
} xk_kcache_format;

/*
 * Indexer logits with the keys in a paged quantized cache.
 *
 * Defines (page "xkernels #27 -- [AMD/MI300A] DeepSeek-V4 DSA indexer +
 * attention", comment announcing dsa_indexer_logits: fp8/fp4 key packing is
 * an encoding of the same dequantized math; page "xkernels #28 --
 * DeepSeek-V4 serving support", comment shipping mxfp4_paged_gather: the
 * paged mxfp4 cache format and its block table): the xk_indexer_logits
 * score with q = e4m3(q8[b,t,h,:]) * q_scale[b,t,h] and key j of sequence b
 * read from page block_table[b, j / bs], row j % bs, dequantized as
 *   XK_KCACHE_MXFP4:        E2M1(nibble d) * E8M0(k_scale byte d/32), 0xFF -> 0
 *                           (element 2i in the low nibble; the gather's format)
 *   XK_KCACHE_FP8_E4M3_OCP: e4m3(k_cache byte d) * k_scale[page, row]
 *
 *   q            [B,T,H,D] OCP e4m3 bytes (16-byte aligned); q_scale [B,T,H] fp32
 *   w            [B,T,H]   fp32 head weights
 *   limit        [B,T]     int32 inclusive last valid position, or NULL (K-1)
 *   k_cache      the pool above (16-byte aligned); k_scale its scales (4-byte aligned)
 *   block_table  [B,MB]    int32 physical page of each logical page
 *   logits       [B,T,K]   fp32 output, -inf past the limit; every element written
 *   bs must be a power of two and K <= MB*bs (else XK_ERR_INVALID_ARGUMENT);
 *   H must be 64, D 128, bs >= 16, NB*bs < 2^31, B*T <= 2^30 and B*T*K <= 2^38 (else
 *   XK_ERR_UNSUPPORTED). Pages holding a valid
 *   position must lie in [0, NB) (not checked on the device).
 */
xk_status xk_indexer_logits_paged(const void* q, const float* q_scale, const float* w,
                                  const int32_t* limit, const void* k_cache, const void* k_scale,
                                  const int32_t* block_table, float* logits, int B, int T, int K,
                                  int H, int D, int MB, int NB, int bs, xk_kcache_format kformat, hipStream_t stream);

/*
 * Bytes of device workspace xk_indexer_topk needs for these sizes (may be 0).
 * Pure host function; returns 0 for sizes xk_indexer_topk would reject.
 */
size_t xk_indexer_topk_workspace_size(int R, int K, int k);

/*
 * Per-row top-k.
 *
 * Defines (page "xkernels #28 -- DeepSeek-V4 serving support": the DSA
 * indexer keeps the top-512 (Flash) / top-1024 (Pro) keys per query; page
 * "DeepSeek V4 Flash on a single AMD MI300X": a deterministic sparse top-k
 * with a tie-break and a canonical order of the selected indices):
 * for row r with n = clamp(limit[r]+1, 0, K) valid keys, idx[r,:] holds the
 * min(k, n) indices j < n with the largest logits[r,j], ordered by
 * (score descending, then lower j), -0.0 equal to +0.0, followed by -1 up to
 * k. The result is unique, so it is bit-reproducible.
 *
 *   logits     [R,K] fp32 (e.g. xk_indexer_logits output with R = B*T)
 *   limit      [R]   int32 inclusive last valid key, or NULL (n = K)
 *   idx        [R,k] int32 output; every element is written
 *   1 <= k <= 2048, else XK_ERR_UNSUPPORTED; K >= 1 (rows up to 16384 keys
 *   are held in registers; longer rows keep a 16384-key prefix there and
 *   stream the rest once).
 *   workspace  device buffer of xk_indexer_topk_workspace_size(R,K,k) bytes
 *              (may be NULL when that size is 0)
 */
xk_status xk_indexer_topk(const float* logits, const int32_t* limit, int32_t* idx,
                          int R, int K, int k,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Sparse attention over the selected rows, read from the paged mxfp4 cache.
 *
 * Defines (page "DeepSeek-V4 on ATOM" tracker, "CSA": the sparse attention
 * path is an index gather, an online softmax and an attention-sink bias;
 * the rows are the ones xk_mxfp4_paged_gather decodes, page "xkernels #28 --
 * DeepSeek-V4 serving support"): with v_j the decoded cache row of slot j
 * (row r's selected position sel_pos[r,j]; slots < 0 take no part), serving
 * as key and value for every head (MQA over the latent row),
 *   s_j        = scale * (q[r,h,:] . v_j)
 *   out[r,h,:] = sum_j exp(s_j) v_j / (sum_j exp(s_j) + exp(sink[h]))
 * and 0 for a row without a valid slot (sink NULL: no sink term).
 *
 *   q            [R,H,D] bf16 (16-byte aligned)
 *   kv_fp4, kv_scale, block_table, sel_pos [R,k], row_seq, S, MB, NB, bs:
 *                as for xk_mxfp4_paged_gather (kv_fp4 16-byte aligned)
 *   sink         [H] fp32 per-head sink logit, or NULL
 *   scale        the softmax scale (finite)
 *   out          [R,H,D] fp32 (16-byte aligned); every element is written
 *   D must be 128, H a multiple of 64 and k <= 2048, else XK_ERR_UNSUPPORTED.
 * Scores and sums are fp32; the weights enter the value sum rounded to bf16
 * (relative error at most 2^-8) while the denominator sums them in fp32, so
 * |out - exact| <= 2^-8 * max_j |v_j| per row, up to fp32 rounding.
 */
xk_status xk_sparse_attention_mxfp4(const void* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                    const int32_t* block_table, const int32_t* sel_pos,
                                    const int32_t* row_seq, const float* sink, float scale,
                                    float* out, int R, int H, int k, int S, int MB, int NB, int bs,
                                    int D, hipStream_t stream);

/*
 * Bytes of device workspace xk_indexer_logits_topk needs for these sizes.
 * Pure host function; returns 0 for sizes xk_indexer_logits_topk would
 * reject. Prefill shapes need about 8 * min(K, 16384) bytes per query plus
 * up to 64 scratch rows of K scores; few-query shapes need the B*T*K scores.
 */
size_t xk_indexer_logits_topk_workspace_size(int B, int T, int K, int k, xk_qk_dtype dtype);

/*
 * Fused indexer logits -> top-k.
 *
 * Defines the composition of the two calls above (page "DeepSeek V4 Flash
 * on a single AMD MI300X", "The patches": a global top-k index preparation
 * for prefill and the deterministic top-k; "Performance", prefill: the
 * deterministic top-k milestone): idx[b*T+t, :] is exactly what
 * xk_indexer_logits followed by xk_indexer_topk (limit read as [B*T])
 * write for the same arguments, element for element, but for prefill
 * shapes without the [B,T,K] score matrix: keys whose score reaches a lower
 * bound on the query's k-th largest score (derived on the fly from scores
 * already seen) are kept as candidates, and the top-k is selected from
 * them. Rows whose candidates overflow their room are rescored and
 * selected from the full row, so the result is exact for any input.
 *
 *   q, q_scale, k, k_scale, w, limit, B, T, K, H, D, dtype: as for
 *               xk_indexer_logits
 *   idx         [B*T, topk] int32 output; every element is written
 *   1 <= topk <= 2048, else XK_ERR_UNSUPPORTED.
 *   workspace   device buffer of at least
 *               xk_indexer_logits_topk_workspace_size(B, T, K, topk, dtype)
 *               bytes, 256-byte aligned; its contents on entry do not
 *               matter and are clobbered. Calls that share a workspace
 *               must be ordered on one stream.
 */
xk_status xk_indexer_logits_topk(const void* q, const float* q_scale,
                                 const void* k, const float* k_scale,
                                 const float* w, const int32_t* limit, int32_t* idx,
                                 int B, int T, int K, int H, int D, int topk, xk_qk_dtype dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused indexer logits -> top-k that allocates nothing, for callers that
 * cannot allocate device memory or cannot pass a workspace (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments and result as xk_indexer_logits_topk, without the workspace:
 * idx is bit-for-bit what xk_indexer_logits_topk writes. Its scratch is a
 * 64 MiB array built into the library (held on every GPU the library runs
 * on until the process ends). Calls needing more are split into slices of
 * whole sequences, or, when one sequence needs more, into ranges of at
 * least 8 of its queries; sizes for which even such a slice needs more
 * than 64 MiB (a sequence of more than ~2M keys) return XK_ERR_UNSUPPORTED
 * before anything is enqueued. The call makes no hipMalloc, hipFree or other
 * allocating call. Every call on one GPU uses that GPU's one array: calls
 * that can overlap on one GPU (different streams, or threads without
 * ordering) race and must not be issued; calls ordered on one stream are
 * safe (nothing in the array needs to start at zero).
 */
xk_status xk_indexer_logits_topk_noalloc(const void* q, const float* q_scale,
                                         const void* k, const float* k_scale,
                                         const float* w, const int32_t* limit, int32_t* idx,
                                         int B, int T, int K, int H, int D, int topk, xk_qk_dtype dtype,
                                         hipStream_t stream);

/*
 * mxfp4 paged KV gather.
 *
 * Defines (page "xkernels #28 -- DeepSeek-V4 serving support", comment
 * shipping mxfp4_paged_gather): for each row r and top-k slot s with
 * p = sel_pos[r,s]:
 *   p < 0  -> out[r,s,:] = 128 x +0.0 (padded slot)
 *   else   -> blk = block_table[row_seq[r], p / bs], off = p % bs and
 *             out[r,s,d] = bf16( E2M1(nibble d) * E8M0(scale byte d/32) )
 * with E8M0(b) = 2^(b-127) and E8M0(0xFF) = 0 (so the product is a signed
 * zero). Every product is exact in bf16 or overflows to +-inf (only for
 * scale bytes >= 253), so the output is bit-exact.
 *
 *   kv_fp4      [NB,bs,D/2] u8  element 2i in the low nibble, 2i+1 in the high
 *   kv_scale    [NB,bs,D/32] u8 E8M0 byte of group g = elements [32g, 32g+32)
 *   block_table [S,MB] int32    physical block of each logical block
 *   sel_pos     [R,k] int32     token positions (e.g. xk_indexer_topk output)
 *   row_seq     [R] int32       sequence of each row, or NULL (row r -> seq r,
 *                               requires R <= S)
 *   out         [R,k,D] bf16 bits (uint16), every element written
 *   bs must be a power of two (else XK_ERR_INVALID_ARGUMENT); D must be
 *   128 and R*k and NB*bs must stay below 2^31, else XK_ERR_UNSUPPORTED;
 *   kv_fp4 must be 4-byte aligned and out 16-byte aligned.
 */
xk_status xk_mxfp4_paged_gather(const uint8_t* kv_fp4, const uint8_t* kv_scale,
                                const int32_t* block_table, const int32_t* sel_pos,
                                const int32_t* row_seq, uint16_t* out,
                                int R, int k, int S, int MB, int NB, int bs, int D,
                                hipStream_t stream);

typedef enum {
  XK_IN_FP32 = 0,  /* float32 rows          */
  XK_IN_BF16 = 1   /* bfloat16 rows (bits)  */
} xk_in_dtype;

/*
 * Per-row OCP fp8 quantizer: the producer of the fp8 q (one row per token
 * and head: per-(token, head) scales) and fp8 k (one row per token).
 *
 * Defines (page "DeepSeek V4 Flash on a single AMD MI300X", "FP8 format"
 * fix: the indexer's fp8 cache is OCP e4m3 written with FP8_MAX = 448; page
 * "DeepSeek-V4 on ATOM", "Quantization & Transform": act_quant bf16 -> fp8
 * e4m3 per 1x128): scale[n] = max_d |x[n,d]| / 448 in fp32 (1 for an
 * all-zero row), out[n,d] = e4m3 round-to-nearest-even of the fp32
 * quotient x[n,d] / scale[n], saturated to +-448.
 *
 *   x      [N,D] fp32 or bf16 (x_dtype), 16-byte aligned
 *   out    [N,D] e4m3 bytes (8-byte aligned); scale [N] fp32
 *   1 <= N <= 2^34, D must be 128 (XK_ERR_UNSUPPORTED otherwise).
 */
xk_status xk_quant_fp8_rows(const void* x, xk_in_dtype x_dtype, uint8_t* out, float* scale, int64_t N, int D,
                            hipStream_t stream);

/*
 * mxfp4 cache writer: rows into the paged mxfp4 cache that
 * xk_mxfp4_paged_gather and xk_indexer_logits_paged read.
 *
 * Defines (the inverse of the gather's decode, page "xkernels #28 --
 * DeepSeek-V4 serving support", comment shipping mxfp4_paged_gather; the
 * rounding is the OCP MX rule, which the pages do not spell out): for row n
 * with slot = slots[n] >= 0 (slot = page * bs + row in page), per 32-element
 * group g: e = floor(log2(max |x|)) - 2 clamped to [-127, 127] (-127 for an
 * all-zero group), kv_scale[slot][g] = e + 127, and element d is the E2M1
 * round-to-nearest-even code of x[n,d] * 2^-e saturated to +-6, element 2i
 * in the low nibble of kv_fp4[slot][i]. Rows with slots[n] < 0 or >= NB*bs
 * are skipped. Rows with equal slots race (last writer wins).
 *
 *   x        [N,D] fp32 or bf16 rows (16-byte aligned); slots [N] int64
 *   kv_fp4   [NB,bs,D/2] u8 (4-byte aligned); kv_scale [NB,bs,D/32] u8 (in place)
 *   1 <= N <= 2^34, D must be 128 (XK_ERR_UNSUPPORTED otherwise).
 */
xk_status xk_mxfp4_cache_write(const void* x, xk_in_dtype x_dtype, const int64_t* slots, uint8_t* kv_fp4,
                               uint8_t* kv_scale, int64_t N, int NB, int bs, int D, hipStream_t stream);

/* Static name of a status code. */
const char* xk_status_string(xk_status status);

/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* xk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XK_H_ */
