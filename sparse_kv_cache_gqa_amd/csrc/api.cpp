// C ABI of libda.so: argument checks on the host, then kernel launches.
// Every check runs before anything is enqueued and touches no HIP state, so
// a rejected call leaves the device and the stream untouched.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "host.h"

namespace da {

namespace {
thread_local char g_err[512] = "";
}

da_status fail(da_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

da_status ok() {
    g_err[0] = '\0';
    return DA_OK;
}

da_status hip_fail(hipError_t e, const char *what) {
    return fail(DA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int esize(int dtype) { return dtype == DA_F32 ? 4 : 2; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
    int r = 0;
    while ((1ll << r) < x) ++r;
    return r;
}

// Checks shared by all attention-shaped calls.  kv4: the cache is uint4 codes
// (kv_dtype is ignored; head_dim must be 128; q is fp32 or fp16).
da_status check_shape(const da_attn_shape *s, bool kv4) {
    if (!s) return fail(DA_E_INVALID, "shape is NULL");
    if (s->batch < 0) return fail(DA_E_INVALID, "batch %d < 0", s->batch);
    if (s->n_kv_heads < 1 || s->n_q_heads < 1)
        return fail(DA_E_INVALID, "head counts must be >= 1 (q %d, kv %d)", s->n_q_heads, s->n_kv_heads);
    if (s->n_q_heads % s->n_kv_heads != 0)
        return fail(DA_E_INVALID, "n_q_heads %d is not a multiple of n_kv_heads %d", s->n_q_heads, s->n_kv_heads);
    const int G = s->n_q_heads / s->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(DA_E_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8}", G);
    if (s->head_dim <= 0) return fail(DA_E_INVALID, "head_dim %d <= 0", s->head_dim);
    if (kv4 ? s->head_dim != 128 : (s->head_dim != 64 && s->head_dim != 128))
        return fail(DA_E_UNSUPPORTED, "head_dim %d not supported", s->head_dim);
    if (s->n_ctx < 1) return fail(DA_E_INVALID, "n_ctx %lld < 1", (long long)s->n_ctx);
    // n_ctx / 16 (the most splits any split size gives) must fit the int32 split count
    if (s->n_ctx > (1ll << 34)) return fail(DA_E_INVALID, "n_ctx %lld > 2^34", (long long)s->n_ctx);
    if (!(s->scale > 0.f) || !isfinite(s->scale)) return fail(DA_E_INVALID, "scale must be finite and > 0");
    if (s->q_dtype < DA_F32 || s->q_dtype > DA_BF16) return fail(DA_E_INVALID, "q_dtype %d", s->q_dtype);
    if (!kv4) {
        if (s->kv_dtype < DA_F32 || s->kv_dtype > DA_BF16) return fail(DA_E_INVALID, "kv_dtype %d", s->kv_dtype);
        if (s->q_dtype != DA_F32 && s->q_dtype != s->kv_dtype)
            return fail(DA_E_UNSUPPORTED, "q_dtype must be fp32 or the KV dtype");
    } else if (s->q_dtype != DA_F32 && s->q_dtype != DA_F16) {
        return fail(DA_E_UNSUPPORTED, "q_dtype must be fp32 or fp16 for a uint4 cache");
    }
    if (s->split_tokens != 0 && (s->split_tokens < 16 || s->split_tokens > 65536 || s->split_tokens % 16 != 0))
        return fail(DA_E_INVALID, "split_tokens %d: 0 or a multiple of 16 in [16, 65536]", s->split_tokens);
    if ((int64_t)s->batch * s->n_kv_heads > 65535)
        return fail(DA_E_UNSUPPORTED, "batch * n_kv_heads %lld > 65535", (long long)s->batch * s->n_kv_heads);
    return DA_OK;
}

int32_t split_tokens_of(const da_attn_shape *s, int mode) {
    if (s->split_tokens) return s->split_tokens;
    return mode == SPLIT_PAGED ? kDefaultSplitPaged
                               : (mode == SPLIT_U4 ? default_split_u4(s->n_ctx, (int64_t)s->batch * s->n_kv_heads)
                                                   : default_split_dense(s->n_ctx));
}

da_status check_ptr(const void *p, const char *name) {
    if (!p) return fail(DA_E_INVALID, "%s is NULL", name);
    if (!aligned16(p)) return fail(DA_E_INVALID, "%s is not 16-byte aligned", name);
    return DA_OK;
}

da_status check_page(int32_t page_size) {
    if (page_size < 1 || page_size > 1024 || !is_pow2(page_size))
        return fail(DA_E_INVALID, "page_size %d: a power of two in [1, 1024]", page_size);
    return DA_OK;
}

int64_t n_pages(const da_attn_shape *s, int32_t page_size) { return (s->n_ctx + page_size - 1) / page_size; }

AttnLaunch dense_launch(const da_attn_shape *s, int kv_fmt, int mode) {
    AttnLaunch a;
    a.B = s->batch;
    a.Hkv = s->n_kv_heads;
    a.G = s->n_q_heads / s->n_kv_heads;
    a.D = s->head_dim;
    a.N = s->n_ctx;
    a.scale_log2 = s->scale * 1.4426950408889634f;
    a.q_fmt = s->q_dtype;
    a.kv_fmt = kv_fmt;
    a.q_bstride = (int64_t)s->n_q_heads * s->head_dim;
    a.o_bstride = (int64_t)s->n_q_heads * s->head_dim;
    a.kv_bstride = (int64_t)s->n_kv_heads * s->n_ctx;
    a.kv_hstride = s->n_ctx;
    a.split_tokens = split_tokens_of(s, mode);
    a.n_split = attn_n_split(s->n_ctx, a.split_tokens, false, 0, 0);
    return a;
}

}  // namespace da

using namespace da;

extern "C" {

int da_version(void) { return (DA_VERSION_MAJOR << 16) | (DA_VERSION_MINOR << 8) | DA_VERSION_PATCH; }

const char *da_status_string(int status) {
    switch (status) {
    case DA_OK: return "DA_OK";
    case DA_E_INVALID: return "DA_E_INVALID";
    case DA_E_UNSUPPORTED: return "DA_E_UNSUPPORTED";
    case DA_E_WORKSPACE: return "DA_E_WORKSPACE";
    case DA_E_NOT_PINNED: return "DA_E_NOT_PINNED";
    case DA_E_HIP: return "DA_E_HIP";
    default: return "unknown da_status";
    }
}

const char *da_last_error(void) { return g_err; }

size_t da_decode_attention_workspace(const da_attn_shape *s) {
    if (check_shape(s, false) != DA_OK) return 0;
    return attn_ws_bytes((int64_t)s->batch * s->n_q_heads,
                         attn_n_split(s->n_ctx, split_tokens_of(s, SPLIT_DENSE), false, 0, 0), s->head_dim);
}

da_status da_decode_attention(const da_attn_shape *s, const void *q, const void *k, const void *v, float *o,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(o, "o"));
    DA_TRY(check_ptr(ws, "ws"));
    const size_t need = da_decode_attention_workspace(s);
    if (ws_bytes < need) return fail(DA_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    AttnLaunch a = dense_launch(s, s->kv_dtype, SPLIT_DENSE);
    if (!attn_supported(a.kv_fmt, a.q_fmt, a.D, a.G, false))
        return fail(DA_E_UNSUPPORTED, "no kernel for this dtype / head_dim / group combination");
    a.q = q;
    a.o = o;
    a.k = k;
    a.v = v;
    a.ws = (float *)ws;
    hipError_t e = launch_attention(a, stream);
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
    return ok();
}

size_t da_decode_attention_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

da_status da_decode_attention_noalloc(const da_attn_shape *s, const void *q, const void *k, const void *v,
                                      float *o, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(o, "o"));
    const size_t need = da_decode_attention_workspace(s);
    if (need > kNoAllocScratchBytes)
        return fail(DA_E_UNSUPPORTED, "this shape needs %zu bytes of split-K scratch, more than the %zu bytes "
                    "the allocation-free entry point holds; use da_decode_attention with a workspace",
                    need, (size_t)kNoAllocScratchBytes);
    AttnLaunch a = dense_launch(s, s->kv_dtype, SPLIT_DENSE);
    if (!attn_supported(a.kv_fmt, a.q_fmt, a.D, a.G, false))
        return fail(DA_E_UNSUPPORTED, "no kernel for this dtype / head_dim / group combination");
    float *scr = nullptr;
    hipError_t e = noalloc_scratch(&scr);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
    a.q = q;
    a.o = o;
    a.k = k;
    a.v = v;
    a.ws = scr;
    e = launch_attention(a, stream);
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
    return ok();
}

da_status da_decode_attention_partials(const da_attn_shape *s, const void *q, const void *k, const void *v,
                                       void *ws, size_t ws_bytes, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(ws, "ws"));
    const size_t need = da_decode_attention_workspace(s);
    if (ws_bytes < need) return fail(DA_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    AttnLaunch a = dense_launch(s, s->kv_dtype, SPLIT_DENSE);
    if (!attn_supported(a.kv_fmt, a.q_fmt, a.D, a.G, false))
        return fail(DA_E_UNSUPPORTED, "no kernel for this dtype / head_dim / group combination");
    a.q = q;
    a.k = k;
    a.v = v;
    a.ws = (float *)ws;
    hipError_t e = launch_split(a, stream);
    if (e != hipSuccess) return hip_fail(e, "partial pass launch");
    return ok();
}

int32_t da_decode_attention_n_split(const da_attn_shape *s) {
    if (check_shape(s, false) != DA_OK) return 0;
    return attn_n_split(s->n_ctx, split_tokens_of(s, SPLIT_DENSE), false, 0, 0);
}

da_status da_merge_partials(int64_t rows, int32_t n_split, int32_t head_dim, const void *partials, float *o,
                            hipStream_t stream) {
    if (rows < 0) return fail(DA_E_INVALID, "rows %lld < 0", (long long)rows);
    if (n_split < 1) return fail(DA_E_INVALID, "n_split %d < 1", n_split);
    if (head_dim != 64 && head_dim != 128) return fail(DA_E_UNSUPPORTED, "head_dim %d not supported", head_dim);
    if (rows > 0x7FFFFFFF) return fail(DA_E_UNSUPPORTED, "rows %lld too many", (long long)rows);
    if (rows == 0) return ok();
    DA_TRY(check_ptr(partials, "partials"));
    DA_TRY(check_ptr(o, "o"));
    hipError_t e = launch_merge(rows, 1, n_split, head_dim, (const float *)partials, o, head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return ok();
}

da_status da_read_stream(const void *buf, uint64_t bytes, int32_t n_groups, uint32_t *sink, hipStream_t stream) {
    if (bytes == 0 || bytes % 16 != 0) return fail(DA_E_INVALID, "bytes %llu: a positive multiple of 16", (unsigned long long)bytes);
    if (bytes > (1ull << 40)) return fail(DA_E_INVALID, "bytes %llu > 2^40", (unsigned long long)bytes);
    if (n_groups < 1 || n_groups > 65535 || (uint64_t)n_groups > bytes / 16)
        return fail(DA_E_INVALID, "n_groups %d: in [1, 65535] and at most bytes / 16", n_groups);
    DA_TRY(check_ptr(buf, "buf"));
    if (!sink) return fail(DA_E_INVALID, "sink is NULL");
    hipError_t e = launch_read_stream(buf, (int64_t)(bytes / 16), n_groups, sink, stream);
    if (e != hipSuccess) return hip_fail(e, "read launch");
    return ok();
}

da_status da_build_page_meta(const da_attn_shape *s, int32_t page_size, const void *k, void *kmin, void *kmax,
                             hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    DA_TRY(check_page(page_size));
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(kmin, "kmin"));
    DA_TRY(check_ptr(kmax, "kmax"));
    hipError_t e = launch_page_meta(s->kv_dtype, (int64_t)s->batch * s->n_kv_heads, s->n_ctx, s->head_dim,
                                    ilog2(page_size), k, kmin, kmax, stream);
    if (e != hipSuccess) return hip_fail(e, "page metadata launch");
    return ok();
}

da_status da_select_pages(const da_attn_shape *s, int32_t page_size, int32_t top_k, const void *q,
                          const void *kmin, const void *kmax, int32_t *page_idx, float *page_score,
                          hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    DA_TRY(check_page(page_size));
    const int64_t P = n_pages(s, page_size);
    if (top_k < 1 || top_k > P) return fail(DA_E_INVALID, "top_k %d not in [1, %lld]", top_k, (long long)P);
    if (P > 8192) return fail(DA_E_UNSUPPORTED, "%lld pages > 8192 per head", (long long)P);
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(kmin, "kmin"));
    DA_TRY(check_ptr(kmax, "kmax"));
    DA_TRY(check_ptr(page_idx, "page_idx"));
    if (page_score && !aligned16(page_score)) return fail(DA_E_INVALID, "page_score is not 16-byte aligned");
    if (!select_supported(s->kv_dtype, s->q_dtype, s->head_dim))
        return fail(DA_E_UNSUPPORTED, "no selection kernel for this dtype / head_dim");
    hipError_t e = launch_select(s->kv_dtype, s->q_dtype, (int64_t)s->batch * s->n_q_heads, s->n_q_heads,
                                 s->n_q_heads / s->n_kv_heads, P, s->head_dim, top_k,
                                 q, kmin, kmax, page_idx, page_score, stream);
    if (e != hipSuccess) return hip_fail(e, "page selection launch");
    return ok();
}

da_status da_select_tokens(const da_attn_shape *s, int32_t top_k, const void *q, const void *k, int32_t *token_idx,
                           float *token_score, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    if (top_k < 1 || top_k > s->n_ctx)
        return fail(DA_E_INVALID, "top_k %d not in [1, %lld]", top_k, (long long)s->n_ctx);
    if (s->n_ctx > 8192) return fail(DA_E_UNSUPPORTED, "%lld tokens > 8192 per head", (long long)s->n_ctx);
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(token_idx, "token_idx"));
    if (token_score && !aligned16(token_score)) return fail(DA_E_INVALID, "token_score is not 16-byte aligned");
    if (!select_supported(s->kv_dtype, s->q_dtype, s->head_dim))
        return fail(DA_E_UNSUPPORTED, "no selection kernel for this dtype / head_dim");
    hipError_t e = launch_select(s->kv_dtype, s->q_dtype, (int64_t)s->batch * s->n_q_heads, s->n_q_heads,
                                 s->n_q_heads / s->n_kv_heads, s->n_ctx, s->head_dim,
                                 top_k, q, k, k, token_idx, token_score, stream, true);
    if (e != hipSuccess) return hip_fail(e, "token selection launch");
    return ok();
}

int64_t da_token_keep_count(int64_t n_ctx) {
    if (n_ctx < 1) return 0;
    // ceil(n_ctx / 10) in integers: no rounding of 0.1 * n_ctx to worry about
    return n_ctx / 10 + (n_ctx % 10 != 0 ? 1 : 0);
}

da_status da_decode_attention_topk(const da_attn_shape *s, int32_t top_k, const void *q, const void *k, const void *v,
                                   float *o, int32_t *token_idx, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    if (top_k < 1 || top_k > s->n_ctx)
        return fail(DA_E_INVALID, "top_k %d not in [1, %lld]", top_k, (long long)s->n_ctx);
    if (s->n_ctx + 2 * (int64_t)top_k + 8 * (int64_t)s->head_dim > 16384)
        return fail(DA_E_UNSUPPORTED, "n_ctx + 2 top_k + 8 head_dim = %lld > 16384",
                    (long long)(s->n_ctx + 2 * (int64_t)top_k + 8 * (int64_t)s->head_dim));
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(o, "o"));
    if (token_idx && !aligned16(token_idx)) return fail(DA_E_INVALID, "token_idx is not 16-byte aligned");
    if (!select_supported(s->kv_dtype, s->q_dtype, s->head_dim))
        return fail(DA_E_UNSUPPORTED, "no selection kernel for this dtype / head_dim");
    hipError_t e = launch_topk_attention(s->kv_dtype, s->q_dtype, (int64_t)s->batch * s->n_q_heads, s->n_q_heads,
                                         s->n_q_heads / s->n_kv_heads, s->n_ctx,
                                         s->head_dim, top_k, s->scale * 1.4426950408889634f, q, k, v, o,
                                         token_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k attention launch");
    return ok();
}

da_status da_decode_attention_sparse(const da_attn_shape *s, int32_t page_size, int32_t top_k, const void *q,
                                     const void *kmin, const void *kmax, const void *k, const void *v, float *o,
                                     int32_t *page_idx, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    DA_TRY(check_page(page_size));
    const int64_t P = n_pages(s, page_size);
    if (top_k < 1 || top_k > P) return fail(DA_E_INVALID, "top_k %d not in [1, %lld]", top_k, (long long)P);
    if (P > 8192) return fail(DA_E_UNSUPPORTED, "%lld pages > 8192 per head", (long long)P);
    const int64_t lds = page_attention_lds_floats(P, top_k, ilog2(page_size), s->head_dim, 16);
    if (lds > kPageAttnLdsFloats)
        return fail(DA_E_UNSUPPORTED, "P + top_k + 2 top_k page_size + 16 head_dim = %lld > %lld", (long long)lds,
                    (long long)kPageAttnLdsFloats);
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(kmin, "kmin"));
    DA_TRY(check_ptr(kmax, "kmax"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(o, "o"));
    if (page_idx && !aligned16(page_idx)) return fail(DA_E_INVALID, "page_idx is not 16-byte aligned");
    if (!select_supported(s->kv_dtype, s->q_dtype, s->head_dim))
        return fail(DA_E_UNSUPPORTED, "no selection kernel for this dtype / head_dim");
    hipError_t e = launch_page_attention(s->kv_dtype, s->q_dtype, (int64_t)s->batch * s->n_q_heads, s->n_q_heads,
                                         s->n_q_heads / s->n_kv_heads, s->n_ctx, P,
                                         s->head_dim, ilog2(page_size), top_k, s->scale * 1.4426950408889634f, q,
                                         kmin, kmax, k, v, o, page_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "page-sparse attention launch");
    return ok();
}

da_status da_prefill_attention(const da_attn_shape *s, int64_t chunk, const void *q, const void *k, const void *v,
                               float *o, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    if (chunk < 1 || chunk > s->n_ctx)
        return fail(DA_E_INVALID, "chunk %lld not in [1, n_ctx = %lld]", (long long)chunk, (long long)s->n_ctx);
    if (s->q_dtype != s->kv_dtype || (s->kv_dtype != DA_BF16 && s->kv_dtype != DA_F16))
        return fail(DA_E_UNSUPPORTED, "prefill needs q and kv both bf16 or both fp16");
    if (!prefill_supported(s->kv_dtype, s->head_dim))
        return fail(DA_E_UNSUPPORTED, "head_dim %d not supported", s->head_dim);
    if (s->n_ctx * (int64_t)s->head_dim * 2 > 0xFFFFFFFFll || chunk * (int64_t)s->head_dim * 2 > 0xFFFFFFFFll)
        return fail(DA_E_UNSUPPORTED, "one head's rows exceed 4 GiB");
    if ((int64_t)s->batch * s->n_q_heads > 65535) return fail(DA_E_UNSUPPORTED, "batch * n_q_heads > 65535");
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(o, "o"));
    hipError_t e = launch_prefill(s->kv_dtype, s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, chunk, s->n_ctx,
                                  s->scale * 1.4426950408889634f, q, k, v, o, stream);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

size_t da_decode_attention_paged_workspace(const da_attn_shape *s, int32_t page_size, int32_t top_k) {
    if (check_shape(s, false) != DA_OK || check_page(page_size) != DA_OK) return 0;
    if (top_k < 1 || top_k > n_pages(s, page_size)) return 0;
    if ((int64_t)s->batch * s->n_q_heads > 65535) return 0;
    const int32_t ns = attn_n_split(s->n_ctx, split_tokens_of(s, SPLIT_PAGED), true, top_k, ilog2(page_size));
    return attn_ws_bytes((int64_t)s->batch * s->n_q_heads, ns, s->head_dim);
}

da_status da_decode_attention_paged(const da_attn_shape *s, int32_t page_size, int32_t top_k,
                                    const int32_t *page_idx, const void *q, const void *k, const void *v, float *o,
                                    void *ws, size_t ws_bytes, hipStream_t stream) {
    DA_TRY(check_shape(s, false));
    DA_TRY(check_page(page_size));
    const int64_t P = n_pages(s, page_size);
    if (top_k < 1 || top_k > P) return fail(DA_E_INVALID, "top_k %d not in [1, %lld]", top_k, (long long)P);
    // one unit per query head: the grid's second dimension is batch * n_q_heads
    if ((int64_t)s->batch * s->n_q_heads > 65535)
        return fail(DA_E_UNSUPPORTED, "batch * n_q_heads %lld > 65535", (long long)s->batch * s->n_q_heads);
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(page_idx, "page_idx"));
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k, "k"));
    DA_TRY(check_ptr(v, "v"));
    DA_TRY(check_ptr(o, "o"));
    DA_TRY(check_ptr(ws, "ws"));
    const size_t need = da_decode_attention_paged_workspace(s, page_size, top_k);
    if (ws_bytes < need) return fail(DA_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    AttnLaunch a = dense_launch(s, s->kv_dtype, SPLIT_PAGED);
    // each query head attends its own pages: one unit per query head
    a.kv_group = a.G;
    a.Hkv = s->n_q_heads;
    a.G = 1;
    if (!attn_supported(a.kv_fmt, a.q_fmt, a.D, a.G, true))
        return fail(DA_E_UNSUPPORTED, "no paged kernel for this dtype / head_dim");
    a.page_idx = page_idx;
    a.top_k = top_k;
    a.log2_page = ilog2(page_size);
    a.n_split = attn_n_split(s->n_ctx, a.split_tokens, true, top_k, a.log2_page);
    a.q = q;
    a.o = o;
    a.k = k;
    a.v = v;
    a.ws = (float *)ws;
    hipError_t e = launch_attention(a, stream);
    if (e != hipSuccess) return hip_fail(e, "paged attention launch");
    return ok();
}

da_status da_quantize_kv4(int64_t n_rows, int32_t row_len, const void *x, uint8_t *codes, void *gmin, void *gscale,
                          hipStream_t stream) {
    if (n_rows < 0) return fail(DA_E_INVALID, "n_rows %lld < 0", (long long)n_rows);
    if (row_len < 64 || row_len % 64 != 0) return fail(DA_E_INVALID, "row_len %d: a positive multiple of 64", row_len);
    if (n_rows == 0) return ok();
    DA_TRY(check_ptr(x, "x"));
    DA_TRY(check_ptr(codes, "codes"));
    DA_TRY(check_ptr(gmin, "gmin"));
    DA_TRY(check_ptr(gscale, "gscale"));
    hipError_t e = launch_quantize_kv4(n_rows * (row_len / 64), x, codes, gmin, gscale, stream);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return ok();
}

da_status da_dequantize_kv4(int64_t n_rows, int32_t row_len, const uint8_t *codes, const void *gmin,
                            const void *gscale, void *x, hipStream_t stream) {
    if (n_rows < 0) return fail(DA_E_INVALID, "n_rows %lld < 0", (long long)n_rows);
    if (row_len < 64 || row_len % 64 != 0) return fail(DA_E_INVALID, "row_len %d: a positive multiple of 64", row_len);
    if (n_rows == 0) return ok();
    DA_TRY(check_ptr(codes, "codes"));
    DA_TRY(check_ptr(gmin, "gmin"));
    DA_TRY(check_ptr(gscale, "gscale"));
    DA_TRY(check_ptr(x, "x"));
    hipError_t e = launch_dequantize_kv4(n_rows * (row_len / 64), codes, gmin, gscale, x, stream);
    if (e != hipSuccess) return hip_fail(e, "dequantize launch");
    return ok();
}

size_t da_decode_attention_kv4_workspace(const da_attn_shape *s) {
    if (check_shape(s, true) != DA_OK) return 0;
    return attn_ws_bytes((int64_t)s->batch * s->n_q_heads,
                         attn_n_split(s->n_ctx, split_tokens_of(s, SPLIT_U4), false, 0, 0), s->head_dim);
}

da_status da_decode_attention_kv4(const da_attn_shape *s, const void *q, const uint8_t *k_codes, const void *k_min,
                                  const void *k_scale, const uint8_t *v_codes, const void *v_min,
                                  const void *v_scale, float *o, void *ws, size_t ws_bytes, hipStream_t stream) {
    DA_TRY(check_shape(s, true));
    if (s->batch == 0) return ok();
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(k_codes, "k_codes"));
    DA_TRY(check_ptr(k_min, "k_min"));
    DA_TRY(check_ptr(k_scale, "k_scale"));
    DA_TRY(check_ptr(v_codes, "v_codes"));
    DA_TRY(check_ptr(v_min, "v_min"));
    DA_TRY(check_ptr(v_scale, "v_scale"));
    DA_TRY(check_ptr(o, "o"));
    DA_TRY(check_ptr(ws, "ws"));
    const size_t need = da_decode_attention_kv4_workspace(s);
    if (ws_bytes < need) return fail(DA_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    AttnLaunch a = dense_launch(s, FMT_U4, SPLIT_U4);
    if (!attn_supported(a.kv_fmt, a.q_fmt, a.D, a.G, false))
        return fail(DA_E_UNSUPPORTED, "no uint4 kernel for this q dtype / group size");
    a.q = q;
    a.o = o;
    a.k = k_codes;
    a.v = v_codes;
    a.kmin = k_min;
    a.kscale = k_scale;
    a.vmin = v_min;
    a.vscale = v_scale;
    a.ws = (float *)ws;
    hipError_t e = launch_attention(a, stream);
    if (e != hipSuccess) return hip_fail(e, "uint4 attention launch");
    return ok();
}

}  // extern "C"
