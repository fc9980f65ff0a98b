/*
 * da.h -- decode attention over a large KV cache on AMD Instinct MI355X
 * (gfx950).  C ABI of libda.so.
 *
 * What is computed
 * ----------------
 * One decode step of attention: for each batch row b and query head j, with
 * KV head h = floor(j / G), G = n_q_heads / n_kv_heads (contiguous groups),
 *
 *     o[b][j] = sum_i softmax_i(scale * q[b][j] . k[b][h][i]) * v[b][h][i]
 *
 * over the cached tokens i (HeadInfer, section "核心 idea", per-head equation;
 * TinyServe, section "方法细节", standard decode step).  Variants:
 *
 *   - da_decode_attention        all N cached tokens (dense).
 *   - da_build_page_meta,        TinyServe's query-aware page selection:
 *     da_select_pages,           per-page per-channel key min/max, the
 *     da_decode_attention_paged  directional bound score, top-K pages, and
 *                                attention over the kept pages only
 *                                (TinyServe, section "方法细节", Algorithm 1).
 *   - da_decode_attention_topk   FlexGen's token-level sparse attention: the
 *     (or da_select_tokens +     top 10% of tokens by exact score q . k, then
 *     da_decode_attention_paged  attention over them only (FlexGen digest,
 *     with page_size 1)          section "方法细节").
 *   - da_quantize_kv4,           FlexGen's 4-bit min/max quantization in
 *     da_dequantize_kv4,         groups of 64 channels, and attention that
 *     da_decode_attention_kv4    dequantizes while loading (FlexGen digest,
 *                                section "方法细节").
 *   - da_prefill_attention       HeadInfer's chunked prefill: a chunk of
 *                                queries attends causally to the cache so far
 *                                and to itself (compute-bound; matrix cores).
 *   - da_stream_*                HeadInfer's head-wise offload: the cache of
 *                                each (layer, KV head) lives in pinned host
 *                                memory and is copied into one of two
 *                                ping-pong device buffers while attention runs
 *                                on the other (HeadInfer, section "方法：
 *                                ping-pong memory 与异步重叠").
 *
 * Conventions (all entry points)
 * ------------------------------
 *   - Memory: every pointer is owned by the caller.  The library allocates no
 *     device or host memory; the split-K workspace is passed in, sized by the
 *     matching *_workspace() call.  da_stream_create allocates only hipEvents.
 *   - Device pointers must be 16-byte aligned; arrays are dense (row-major,
 *     last index fastest) in the layouts given below.
 *   - dtypes: q and K/V are fp32, fp16 or bf16 (DA_F32/DA_F16/DA_BF16); the
 *     output is always fp32.  q must be fp32 or the KV dtype.
 *   - Errors: every argument is checked on the host before anything is
 *     enqueued.  On an error nothing is launched, a da_status is returned and
 *     da_last_error() holds a message (thread-local).  DA_OK means enqueued:
 *     the work is asynchronous on the given stream, and device faults surface
 *     at the caller's next synchronisation.
 *   - Streams: hipStream_t values (0 = the null stream).  Calls on one stream
 *     run in order; calls that share a workspace must not overlap.
 *   - Reentrancy: entry points keep no state between calls except
 *     da_stream_ctx objects, which must not be shared by concurrent calls.
 */
#ifndef DA_H
#define DA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef DA_HIP_STREAM_DEFINED
#define DA_HIP_STREAM_DEFINED
typedef struct ihipStream_t *hipStream_t;
#endif

#define DA_VERSION_MAJOR 0
#define DA_VERSION_MINOR 1
#define DA_VERSION_PATCH 0

typedef enum da_status {
    DA_OK = 0,
    DA_E_INVALID = 1,      /* null/misaligned pointer, bad size or index  */
    DA_E_UNSUPPORTED = 2,  /* valid but not built: head_dim, dtype, G ... */
    DA_E_WORKSPACE = 3,    /* ws_bytes smaller than the *_workspace size  */
    DA_E_NOT_PINNED = 4,   /* host pointer not in page-locked memory      */
    DA_E_HIP = 5           /* a HIP runtime call failed (see last_error)  */
} da_status;

typedef enum da_dtype { DA_F32 = 0, DA_F16 = 1, DA_BF16 = 2 } da_dtype;

/* Shape of one decode-attention call.
 *   batch >= 1; n_kv_heads >= 1; n_q_heads = G * n_kv_heads with
 *   G in {1, 2, 4, 8}; head_dim in {64, 128}; 1 <= n_ctx <= 2^34 tokens per
 *   (batch row, KV head); scale > 0 (normally 1/sqrt(head_dim)); q_dtype is DA_F32
 *   or kv_dtype; split_tokens is the number of tokens (dense) or selected
 *   token positions (paged) one workgroup reduces before the cross-split
 *   merge: 0 selects the entry point's default (dense and head-wise: the
 *   power of two nearest above n_ctx/16 within [256, 2048]; paged 512;
 *   uint4: the longest power of two from 256 that still gives at least
 *   2048 (split, batch row, KV head) waves); otherwise a multiple of 16 in
 *   [16, 65536].  The dense, head-wise and paged splits never depend on
 *   batch or head counts, so there a call over one head and a call over all
 *   heads give bitwise-equal results for that head. */
typedef struct da_attn_shape {
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int64_t n_ctx;
    float   scale;
    int32_t q_dtype;       /* da_dtype */
    int32_t kv_dtype;      /* da_dtype */
    int32_t split_tokens;
} da_attn_shape;

/* (DA_VERSION_MAJOR << 16) | (DA_VERSION_MINOR << 8) | DA_VERSION_PATCH */
int da_version(void);
const char *da_status_string(int status);
/* Message for the last non-OK status returned on this thread ("" if none). */
const char *da_last_error(void);

/* ------------------------------------------------------------------------
 * Dense decode attention (HeadInfer per-head equation; TinyServe Attn(q,K,V))
 *   q  [batch][n_q_heads][head_dim]          q_dtype, device
 *   k  [batch][n_kv_heads][n_ctx][head_dim]  kv_dtype, device
 *   v  same layout as k
 *   o  [batch][n_q_heads][head_dim]          fp32, device (written)
 *   ws >= da_decode_attention_workspace(s) bytes, device scratch holding the
 *      per-split (max, sum, unnormalised output) partials; contents on entry
 *      are ignored.
 * Two kernels on `stream`: a split-K partial pass and a cross-split merge.
 * When there is one split, or at most four splits per (batch row, KV head)
 * with at least 256 such units and at most 4096 splits in all, the splits of
 * a unit instead run as the waves of one workgroup and merge in LDS: one
 * kernel, the same result bit for bit, and ws is not written.  The same rule
 * holds for the paged, uint4 and head-wise entry points.
 * ------------------------------------------------------------------------ */
size_t da_decode_attention_workspace(const da_attn_shape *s);
da_status da_decode_attention(const da_attn_shape *s, const void *q,
                              const void *k, const void *v, float *o,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * da_decode_attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  Same kernels, split and result bit for bit as
 * da_decode_attention; the split-K partials go to a fixed array of
 * da_decode_attention_noalloc_max_scratch() bytes (16 MiB) that the library
 * holds on each GPU it runs on until the process ends.  A shape whose
 * da_decode_attention_workspace exceeds that size is refused with
 * DA_E_UNSUPPORTED (nothing enqueued).  The call allocates nothing (no
 * hipMalloc or hipFree); the first call on a device looks up the array's
 * device address once.  Every call on one GPU shares that array: calls that
 * may overlap on one GPU (different streams, or host threads without
 * ordering) race and must not be issued; calls ordered on one stream are
 * safe.  Nothing in the array needs to start zeroed.
 * ------------------------------------------------------------------------ */
size_t da_decode_attention_noalloc_max_scratch(void);
da_status da_decode_attention_noalloc(const da_attn_shape *s, const void *q,
                                      const void *k, const void *v, float *o,
                                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * The two halves of da_decode_attention, for callers that merge partials
 * themselves (for example partials computed over different token ranges, on
 * different devices, of one sequence) or time the passes apart.
 *
 * da_decode_attention_partials: the split-K pass only.  Writes, for every
 *   query-head row r = b * n_q_heads + j and split i (tokens
 *   [i * split, min((i+1) * split, n_ctx)), split = split_tokens or the
 *   dense default above),
 *   ws[r][i][0..head_dim+3] fp32 = (u[0..head_dim-1], m, l, pad, pad)
 *   with m = max_t x_t, l = sum_t 2^(x_t - m), u = sum_t 2^(x_t - m) v_t and
 *   x_t = scale * log2(e) * q . k_t (base-2 logits).  n_split is
 *   da_decode_attention_n_split(s); ws as for da_decode_attention.
 * da_merge_partials: o[r] = sum_i 2^(m_i - M) u_i / sum_i 2^(m_i - M) l_i,
 *   M = max_i m_i, for rows r < rows, partials [rows][n_split][head_dim+4]
 *   fp32 (device), o [rows][head_dim] fp32 (device).  A split with
 *   m = -inf contributes nothing; a row whose splits all have m = -inf
 *   (no token) gets o = 0.  head_dim in {64, 128}.
 * ------------------------------------------------------------------------ */
int32_t da_decode_attention_n_split(const da_attn_shape *s);
da_status da_decode_attention_partials(const da_attn_shape *s, const void *q,
                                       const void *k, const void *v, void *ws,
                                       size_t ws_bytes, hipStream_t stream);
da_status da_merge_partials(int64_t rows, int32_t n_split, int32_t head_dim,
                            const void *partials, float *o, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Page metadata (TinyServe phi(K_j) = (m_j, M_j)): per page of page_size
 * tokens, the per-channel minimum and maximum of the keys.  Page j covers
 * tokens [j*page_size, min((j+1)*page_size, n_ctx)); P = ceil(n_ctx/page_size).
 *   k     [batch][n_kv_heads][n_ctx][head_dim] kv_dtype, device
 *   kmin, kmax [batch][n_kv_heads][P][head_dim] kv_dtype, device (written)
 * page_size: a power of two in [1, 1024].  Exact (no rounding).
 * ------------------------------------------------------------------------ */
da_status da_build_page_meta(const da_attn_shape *s, int32_t page_size,
                             const void *k, void *kmin, void *kmax,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * Query-aware page selection (TinyServe relevance score and S_t = TopK):
 *   r_j = sum_d (q_d * kmax[j][d] if q_d >= 0 else q_d * kmin[j][d])
 * accumulated in fp32 (products of fp16/bf16 values are exact in fp32), then
 * the top_k largest r_j per (batch row, query head); equal scores keep the
 * lower page index; the kept indices are written in ascending order.  With
 * grouped-query heads each query head j selects its own pages over the
 * metadata of its KV head j / (n_q_heads / n_kv_heads).
 *   q          [batch][n_q_heads][head_dim]   q_dtype, device
 *   kmin, kmax as written by da_build_page_meta ([batch][n_kv_heads][P][D])
 *   page_idx   [batch][n_q_heads][top_k] int32, device (written)
 *   page_score [batch][n_q_heads][P] fp32, device, or NULL (written if given)
 * Requires 1 <= top_k <= P, P <= 8192, page_size a power of two in [1, 1024].
 * ------------------------------------------------------------------------ */
da_status da_select_pages(const da_attn_shape *s, int32_t page_size,
                          int32_t top_k, const void *q, const void *kmin,
                          const void *kmax, int32_t *page_idx,
                          float *page_score, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Token selection by exact score (FlexGen's top-10% sparse attention keeps,
 * per query, the indices of its best-scoring keys):
 *   s_i = q . k_i accumulated in fp32 (products of fp16/bf16 values exact),
 * then the top_k largest s_i per (batch row, query head), k_i being the keys
 * of the query head's KV head; equal scores keep the lower token index; the
 * kept indices are written in ascending order.  Reads each key row once per
 * query head.  Attention over the kept tokens is da_decode_attention_paged
 * with page_size 1 and page_idx = token_idx.
 *   q           [batch][n_q_heads][head_dim]          q_dtype, device
 *   k           [batch][n_kv_heads][n_ctx][head_dim]  kv_dtype, device
 *   token_idx   [batch][n_q_heads][top_k] int32, device (written)
 *   token_score [batch][n_q_heads][n_ctx] fp32, device, or NULL (written if
 *               given; unscaled q . k)
 * Requires 1 <= top_k <= n_ctx <= 8192.
 * ------------------------------------------------------------------------ */
da_status da_select_tokens(const da_attn_shape *s, int32_t top_k,
                           const void *q, const void *k, int32_t *token_idx,
                           float *token_score, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Number of tokens FlexGen's sparse attention keeps per query (FlexGen
 * digest, section "方法细节": only the top 10% of the K cache by score are
 * kept): ceil(n_ctx / 10), which is at least 1 and at most n_ctx for
 * n_ctx >= 1.  Returns 0 when n_ctx < 1.  Pure host arithmetic (integer, no
 * rounding); pass the result as top_k to da_select_tokens or
 * da_decode_attention_topk.
 * ------------------------------------------------------------------------ */
int64_t da_token_keep_count(int64_t n_ctx);

/* ------------------------------------------------------------------------
 * Token-level top-k sparse attention in one kernel (FlexGen's top-10% sparse
 * attention): per (batch row, query head) the exact scores s_i = q . k_i of
 * all n_ctx tokens of its KV head, the top_k of them (as da_select_tokens),
 * then
 *   o = sum_i softmax(scale * s_i) v_i over the kept tokens only,
 * reading only the value rows of the kept tokens.  No workspace.
 *   q, k, v, o  as for da_decode_attention
 *   token_idx   [batch][n_q_heads][top_k] int32, device, or NULL (written if
 *               given: the kept tokens, ascending)
 * Requires 1 <= top_k <= n_ctx and n_ctx + 2 top_k + 8 head_dim <= 16384
 * (the scores, the kept list and its weights stay in LDS).
 * ------------------------------------------------------------------------ */
da_status da_decode_attention_topk(const da_attn_shape *s, int32_t top_k,
                                   const void *q, const void *k, const void *v,
                                   float *o, int32_t *token_idx,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse attention over the selected pages only (TinyServe SparseAttn):
 * softmax normalised over the tokens of the listed pages; positions at or
 * beyond n_ctx in a partial last page are skipped, and so is any listed page
 * index outside [0, P).  A row whose list holds no page inside [0, P) has
 * no token to attend, and its output is zero.  Each query head attends its
 * own list over the rows of its KV head (grouped-query heads: one list per
 * query head).  batch * n_q_heads <= 65535 (DA_E_UNSUPPORTED otherwise).
 *   page_idx [batch][n_q_heads][top_k] int32, device
 *   q, k, v, o as for da_decode_attention
 *   ws >= da_decode_attention_paged_workspace(s, page_size, top_k) bytes
 * ------------------------------------------------------------------------ */
size_t da_decode_attention_paged_workspace(const da_attn_shape *s,
                                           int32_t page_size, int32_t top_k);
da_status da_decode_attention_paged(const da_attn_shape *s, int32_t page_size,
                                    int32_t top_k, const int32_t *page_idx,
                                    const void *q, const void *k, const void *v,
                                    float *o, void *ws, size_t ws_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * TinyServe's whole decode step for one query (its Algorithm 1: given q, the
 * page metadata and the KV cache, return o) in one kernel: per (batch row,
 * query head) the bound scores of all pages of its KV head (as
 * da_select_pages), the top_k of them, the exact scores q . k of the tokens
 * of the kept pages, and
 *   o = sum_t softmax(scale * q . k_t) v_t over those tokens only
 * (as da_decode_attention_paged on the same page list; positions at or beyond
 * n_ctx in a partial last page are skipped).  Reads the metadata once and
 * only the kept pages' K and V rows.  No workspace.
 *   q, k, v, o   as for da_decode_attention
 *   kmin, kmax   as written by da_build_page_meta with this page_size
 *   page_idx     [batch][n_q_heads][top_k] int32, device, or NULL (written
 *                if given: the kept pages, ascending, as da_select_pages)
 * Requires 1 <= top_k <= P = ceil(n_ctx / page_size) <= 8192 and
 * P + top_k + 2 top_k page_size + 16 head_dim <= 16384 (page scores, the
 * kept list and two floats per kept token stay in LDS); DA_E_UNSUPPORTED
 * otherwise.
 * ------------------------------------------------------------------------ */
da_status da_decode_attention_sparse(const da_attn_shape *s, int32_t page_size,
                                     int32_t top_k, const void *q,
                                     const void *kmin, const void *kmax,
                                     const void *k, const void *v, float *o,
                                     int32_t *page_idx, hipStream_t stream);

/* ------------------------------------------------------------------------
 * uint4 group quantization (FlexGen 4-bit, groups of 64 along the hidden
 * dimension).  For each row and each group of 64 contiguous fp16 values:
 *   min = minimum, max = maximum,
 *   scale = fp16((max - min) / 15)     exact quotient rounded once (RNE),
 *   code  = clamp(round_half_even((x - min) / scale), 0, 15), 0 if scale == 0,
 * two codes per byte, even channel in the low nibble.  Bit-exact.
 *   x      [n_rows][row_len] fp16, device (row_len a multiple of 64)
 *   codes  [n_rows][row_len/2] uint8, device (written)
 *   gmin, gscale [n_rows][row_len/64] fp16, device (written)
 * da_dequantize_kv4 writes x_hat = fp16(min + code * scale), rounded once.
 * ------------------------------------------------------------------------ */
da_status da_quantize_kv4(int64_t n_rows, int32_t row_len, const void *x,
                          uint8_t *codes, void *gmin, void *gscale,
                          hipStream_t stream);
da_status da_dequantize_kv4(int64_t n_rows, int32_t row_len,
                            const uint8_t *codes, const void *gmin,
                            const void *gscale, void *x, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode attention over a uint4 cache, dequantizing while loading (FlexGen
 * digest, section "方法细节": the KV cache is stored as 4-bit integers with
 * a min and a scale per group of 64 along the hidden dimension, and is
 * dequantized back to FP16 before the attention arithmetic).  Per (batch
 * row, query head) it computes the dense output above over the dequantized
 * keys and values x_hat = min + code * scale of its KV head.
 * The dequantization is folded into the fp32 arithmetic
 * (q . (min + c*scale) = min * sum(q) + scale * sum(q*c) per group, and the
 * same for the value side), which differs from rounding each dequantized
 * element to fp16 first by at most half an fp16 ulp per element.
 *   q                 [batch][n_q_heads][head_dim]  fp16 or fp32, device
 *   k_codes, v_codes  [batch][n_kv_heads][n_ctx][head_dim/2] uint8, device
 *   k_min, k_scale, v_min, v_scale
 *                     [batch][n_kv_heads][n_ctx][head_dim/64] fp16, device
 *   o                 [batch][n_q_heads][head_dim] fp32, device (written)
 * head_dim must be 128; kv_dtype is ignored; ws as reported.  A query head
 * holding a NaN or an infinity gets an unspecified row of o; the other rows
 * are unaffected.
 * ------------------------------------------------------------------------ */
size_t da_decode_attention_kv4_workspace(const da_attn_shape *s);
da_status da_decode_attention_kv4(const da_attn_shape *s, const void *q,
                                  const uint8_t *k_codes, const void *k_min,
                                  const void *k_scale, const uint8_t *v_codes,
                                  const void *v_min, const void *v_scale,
                                  float *o, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * Chunked prefill attention (HeadInfer, section "chunked prefill 与 adaptive
 * head grouping"): a chunk of `chunk` queries at positions
 * prefix .. prefix + chunk - 1, prefix = n_ctx - chunk, attends causally:
 *   o[b][j][i] = sum_{t <= prefix + i} softmax_t(scale * q[b][j][i] . k[b][h][t]) v[b][h][t]
 * with h = floor(j / G).  The cache rows of the chunk itself must already be
 * in k and v (n_ctx = prefix + chunk rows).  Matrix-core products with fp32
 * accumulation; the probabilities enter the second product as two 16-bit
 * terms (about 2^-16 relative each).
 *   q [batch][n_q_heads][chunk][head_dim]   q_dtype == kv_dtype, bf16 or fp16
 *   k, v [batch][n_kv_heads][n_ctx][head_dim]
 *   o [batch][n_q_heads][chunk][head_dim]   fp32, device (written)
 * Requires 1 <= chunk <= n_ctx, head_dim in {64, 128}, batch * n_q_heads
 * <= 65535.  No workspace.
 * ------------------------------------------------------------------------ */
da_status da_prefill_attention(const da_attn_shape *s, int64_t chunk,
                               const void *q, const void *k, const void *v,
                               float *o, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Head-wise streamed decode (HeadInfer).
 * `per_layer` describes one layer (batch, heads, head_dim, n_ctx, dtypes).
 * heads_per_chunk (1, 2, 4 or 8, dividing n_kv_heads) KV heads are copied
 * per transfer (HeadInfer's adaptive head grouping; n_kv_heads = layer-wise).
 *
 * da_headwise_buffer_bytes: bytes of ONE ping-pong buffer, i.e. K and V of
 *   heads_per_chunk heads: 2 * heads_per_chunk * batch * n_ctx * head_dim *
 *   sizeof(kv).  Pure host arithmetic.
 * da_stream_headwise: for each layer l and chunk c (in order), on `copy`:
 *   wait until the buffer's previous attention finished, copy K then V of
 *   the chunk's heads from pinned host memory into buffer (chunk index % 2);
 *   on `compute`: wait for the copy, run attention for those heads.
 *   k_host[l * n_kv_heads + h], v_host[...]: [batch][n_ctx][head_dim]
 *     kv_dtype in page-locked host memory (hipHostMalloc), one per
 *     (layer, KV head);
 *   buf0, buf1: device buffers of da_stream_buffer_bytes each;
 *   q [n_layers][batch][n_q_heads][head_dim] q_dtype, device;
 *   o [n_layers][batch][n_q_heads][head_dim] fp32, device (written);
 *   ws >= da_stream_workspace(ctx) bytes, device (that size covers every
 *     attended length 1..n_ctx, so it stays valid as the length changes);
 *   compute != copy.  The output is complete when `compute` drains.
 * Each head's result is bitwise equal to da_decode_attention on the same
 * data with the same split_tokens.
 *
 * Growing the context (the per-step append of the new token's K/V; HeadInfer
 * keeps the whole cache on the host):  the n_ctx of `per_layer` is the row
 * capacity `cap` of every host cache ([batch][cap][head_dim]); a context
 * attends to the first `len` rows of each batch row (len = cap at creation,
 * da_stream_length / da_stream_set_length, 1 <= len <= cap), copying them
 * into a dense [batch][len][head_dim] buffer; the attention then equals
 * da_decode_attention over those len tokens.
 * da_stream_append: on `stream`, writes the new token's rows
 *   k_new, v_new [n_layers][batch][n_kv_heads][head_dim] kv_dtype, device,
 * into row len of every host cache (head_dim values per (layer, head, batch
 * row)) with one kernel per 32 layer-heads that stores to the page-locked
 * caches directly, then sets len = len + 1 on the host.  Fails with
 * DA_E_INVALID when len == cap, and with DA_E_NOT_PINNED (nothing enqueued)
 * unless every cache is page-locked host memory that the device maps at its
 * host address (hipHostMalloc).  The rows are in host memory once the
 * kernels have completed; give it the copy stream of the next
 * da_stream_headwise (or order the streams), so the rows land first.
 * ------------------------------------------------------------------------ */
typedef struct da_stream_ctx da_stream_ctx;

size_t da_headwise_buffer_bytes(const da_attn_shape *per_layer,
                                int32_t heads_per_chunk);
da_status da_stream_create(const da_attn_shape *per_layer,
                           int32_t heads_per_chunk, da_stream_ctx **out);
size_t da_stream_buffer_bytes(const da_stream_ctx *c);
size_t da_stream_workspace(const da_stream_ctx *c);
da_status da_stream_headwise(da_stream_ctx *c, int32_t n_layers,
                             const void *const *k_host,
                             const void *const *v_host, void *buf0, void *buf1,
                             const void *q, float *o, void *ws,
                             size_t ws_bytes, hipStream_t compute,
                             hipStream_t copy);
int64_t da_stream_length(const da_stream_ctx *c);
da_status da_stream_set_length(da_stream_ctx *c, int64_t len);
da_status da_stream_append(da_stream_ctx *c, int32_t n_layers,
                           const void *k_new, const void *v_new,
                           void *const *k_host, void *const *v_host,
                           hipStream_t stream);
void da_stream_destroy(da_stream_ctx *c);

/* ------------------------------------------------------------------------
 * Measurement aid (not part of the attention method): the practical HBM read
 * bandwidth that the decode kernels' byte rates are set against, beside the
 * published peak.  da_read_stream reads `bytes` (a positive multiple of 16,
 * at most 2^40) of device memory at `buf` (16-byte aligned) exactly once with
 * non-temporal 16-byte loads, as n_groups single-wave workgroups (1..65535,
 * at most bytes/16) that each stream one contiguous chunk of
 * floor(bytes/16/n_groups) 16-byte units (the last also takes the rest), and
 * writes the XOR of each chunk's 32-bit words to sink[g] (device, n_groups
 * uint32, caller-owned).  Bad arguments: DA_E_INVALID; launch failure:
 * DA_E_HIP.  Asynchronous on `stream`.
 * ------------------------------------------------------------------------ */
da_status da_read_stream(const void *buf, uint64_t bytes, int32_t n_groups,
                         uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DA_H */
