// Head-wise streamed decode (HeadInfer, section "方法：ping-pong memory 与异步
// 重叠"): only the KV cache of the heads being computed is resident.  Two
// device buffers alternate: while attention runs on one (compute stream), the
// next chunk of heads is copied host-to-device into the other (copy stream).
// Ordering uses two events per buffer: `ready` (copy done -> compute may
// start) and `freed` (compute done -> the buffer may be overwritten).  Every
// copy into a buffer waits for that buffer's last `freed`, also across calls,
// so back-to-back calls on one context need no ordering by the caller.
//
// HeadInfer also writes the previous head back device-to-host; a decode step
// does not change the cached keys and values, so there is nothing to write
// back and that copy is not issued.  What a step does add is the new token:
// da_stream_append writes its key and value rows (head_dim values per head
// and batch row) into row `len` of every host cache, with a kernel that
// stores to the page-locked caches directly, and extends the attended
// length.  The host caches hold `cap` rows per batch row
// (the n_ctx given at creation); a step streams the first `len` rows of each
// batch row into a dense [batch][len][head_dim] buffer.
#include "host.h"
#include "append.h"

#include <algorithm>
#include <new>

struct da_stream_ctx {
    da_attn_shape shape;     // n_ctx = cap, the host caches' rows per batch row
    int64_t len;             // rows attended (and copied) per batch row, <= cap
    int32_t hpc;             // heads per chunk (per transfer)
    int device;
    hipEvent_t ready[2];
    hipEvent_t freed[2];
    // freed[i] has been recorded (by this call or an earlier one): every
    // later copy into buffer i must wait for it, including the first two
    // copies of the next call, whose buffers the previous call's last two
    // attentions may still be reading
    bool freed_recorded[2];
};

namespace da {
namespace {

size_t head_bytes(const da_attn_shape *s) {
    return (size_t)s->batch * (size_t)s->n_ctx * (size_t)s->head_dim * (size_t)esize(s->kv_dtype);
}

da_status check_hpc(const da_attn_shape *s, int32_t hpc) {
    if (hpc != 1 && hpc != 2 && hpc != 4 && hpc != 8)
        return fail(DA_E_INVALID, "heads_per_chunk %d not in {1,2,4,8}", hpc);
    if (s->n_kv_heads % hpc != 0)
        return fail(DA_E_INVALID, "heads_per_chunk %d does not divide n_kv_heads %d", hpc, s->n_kv_heads);
    return DA_OK;
}

// Page-locked host memory; with `mapped`, also mapped at the same address on
// the device.
da_status check_pinned(const void *p, const char *name, int64_t idx, bool mapped = false) {
    if (!p) return fail(DA_E_INVALID, "%s[%lld] is NULL", name, (long long)idx);
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(DA_E_NOT_PINNED, "%s[%lld] is not page-locked host memory (%s)", name, (long long)idx,
                    hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeHost)
        return fail(DA_E_NOT_PINNED, "%s[%lld] is not page-locked host memory", name, (long long)idx);
    if (mapped) {
        // kernels store to such memory at its host address (one virtual
        // address space for host and device); anything else is refused
        if (!attr.hostPointer || attr.hostPointer != attr.devicePointer)
            return fail(DA_E_NOT_PINNED, "%s[%lld] is not mapped at its host address on the device", name,
                        (long long)idx);
    }
    return DA_OK;
}

}  // namespace
}  // namespace da

using namespace da;

extern "C" {

size_t da_headwise_buffer_bytes(const da_attn_shape *s, int32_t heads_per_chunk) {
    if (check_shape(s, false) != DA_OK || check_hpc(s, heads_per_chunk) != DA_OK) return 0;
    return 2 * (size_t)heads_per_chunk * head_bytes(s);
}

da_status da_stream_create(const da_attn_shape *s, int32_t heads_per_chunk, da_stream_ctx **out) {
    if (!out) return fail(DA_E_INVALID, "out is NULL");
    *out = nullptr;
    DA_TRY(check_shape(s, false));
    DA_TRY(check_hpc(s, heads_per_chunk));
    if (s->batch < 1) return fail(DA_E_INVALID, "batch must be >= 1 for streaming");
    const int G = s->n_q_heads / s->n_kv_heads;
    if (!attn_supported(s->kv_dtype, s->q_dtype, s->head_dim, G, false))
        return fail(DA_E_UNSUPPORTED, "no kernel for this dtype / head_dim / group combination");
    auto *c = new (std::nothrow) da_stream_ctx();
    if (!c) return fail(DA_E_INVALID, "out of host memory");
    c->shape = *s;
    c->len = s->n_ctx;
    c->hpc = heads_per_chunk;
    hipError_t e = hipGetDevice(&c->device);
    int made = 0;
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
        e = hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming);
        if (e == hipSuccess) ++made;
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->freed[i], hipEventDisableTiming);
        if (e == hipSuccess) ++made;
    }
    if (e != hipSuccess) {
        for (int i = 0; i < made; ++i) (void)hipEventDestroy(i % 2 == 0 ? c->ready[i / 2] : c->freed[i / 2]);
        delete c;
        return hip_fail(e, "stream context events");
    }
    *out = c;
    return ok();
}

size_t da_stream_buffer_bytes(const da_stream_ctx *c) {
    return c ? 2 * (size_t)c->hpc * head_bytes(&c->shape) : 0;
}

size_t da_stream_workspace(const da_stream_ctx *c) {
    if (!c) return 0;
    const da_attn_shape *s = &c->shape;
    const int G = s->n_q_heads / s->n_kv_heads;
    // a step attends len <= cap tokens, split by len's own split size, and
    // the default split grows in steps with the length: the most splits over
    // 1 <= len <= cap come at cap or at the last length of a smaller split
    int32_t most = 0;
    for (int64_t len = 1; len <= s->n_ctx; len *= 2) {
        da_attn_shape t = *s;
        t.n_ctx = len;
        most = std::max(most, attn_n_split(len, split_tokens_of(&t, SPLIT_DENSE), false, 0, 0));
    }
    most = std::max(most, attn_n_split(s->n_ctx, split_tokens_of(s, SPLIT_DENSE), false, 0, 0));
    return attn_ws_bytes((int64_t)s->batch * c->hpc * G, most, s->head_dim);
}

da_status da_stream_headwise(da_stream_ctx *c, int32_t n_layers, const void *const *k_host,
                             const void *const *v_host, void *buf0, void *buf1, const void *q, float *o, void *ws,
                             size_t ws_bytes, hipStream_t compute, hipStream_t copy) {
    if (!c) return fail(DA_E_INVALID, "context is NULL");
    if (n_layers < 1) return fail(DA_E_INVALID, "n_layers %d < 1", n_layers);
    if (!k_host || !v_host) return fail(DA_E_INVALID, "host pointer arrays are NULL");
    if (compute == copy) return fail(DA_E_INVALID, "compute and copy streams must differ");
    const da_attn_shape *s = &c->shape;
    DA_TRY(check_ptr(buf0, "buf0"));
    DA_TRY(check_ptr(buf1, "buf1"));
    DA_TRY(check_ptr(q, "q"));
    DA_TRY(check_ptr(o, "o"));
    DA_TRY(check_ptr(ws, "ws"));
    if (ws_bytes < da_stream_workspace(c))
        return fail(DA_E_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, da_stream_workspace(c));
    const int64_t n_heads = (int64_t)n_layers * s->n_kv_heads;
    for (int64_t i = 0; i < n_heads; ++i) {
        DA_TRY(check_pinned(k_host[i], "k_host", i));
        DA_TRY(check_pinned(v_host[i], "v_host", i));
    }

    const int G = s->n_q_heads / s->n_kv_heads;
    da_attn_shape cur = *s;                       // the attended length
    cur.n_ctx = c->len;
    const size_t hb = head_bytes(&cur);           // bytes of one head's K (or V) in a buffer
    const size_t row_dev = (size_t)c->len * s->head_dim * esize(s->kv_dtype);
    const size_t row_host = (size_t)s->n_ctx * s->head_dim * esize(s->kv_dtype);
    const int n_chunks = s->n_kv_heads / c->hpc;
    const int qes = esize(s->q_dtype);
    AttnLaunch a = dense_launch(&cur, s->kv_dtype, SPLIT_DENSE);
    a.Hkv = c->hpc;
    a.kv_bstride = c->len;                        // buffer layout [hpc][B][len][D]
    a.kv_hstride = (int64_t)s->batch * c->len;
    // host rows [B][cap][D] -> device [B][len][D]: one copy when len == cap
    auto h2d = [&](void *dst, const void *src) -> hipError_t {
        if (row_dev == row_host) return hipMemcpyAsync(dst, src, hb, hipMemcpyHostToDevice, copy);
        return hipMemcpy2DAsync(dst, row_dev, src, row_host, row_dev, (size_t)s->batch, hipMemcpyHostToDevice,
                                copy);
    };
    a.ws = (float *)ws;
    void *bufs[2] = {buf0, buf1};

    hipError_t e = hipSuccess;
    for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
        for (int ch = 0; ch < n_chunks && e == hipSuccess; ++ch) {
            const int64_t u = (int64_t)l * n_chunks + ch;
            const int slot = (int)(u & 1);
            char *kb = (char *)bufs[slot];
            char *vb = kb + (size_t)c->hpc * hb;
            if (c->freed_recorded[slot]) e = hipStreamWaitEvent(copy, c->freed[slot], 0);
            for (int i = 0; i < c->hpc && e == hipSuccess; ++i) {
                const int64_t hi = (int64_t)l * s->n_kv_heads + (int64_t)ch * c->hpc + i;
                e = h2d(kb + i * hb, k_host[hi]);
                if (e == hipSuccess) e = h2d(vb + i * hb, v_host[hi]);
            }
            if (e == hipSuccess) e = hipEventRecord(c->ready[slot], copy);
            if (e == hipSuccess) e = hipStreamWaitEvent(compute, c->ready[slot], 0);
            if (e != hipSuccess) break;
            const int64_t head0 = ((int64_t)l * s->batch * s->n_q_heads + (int64_t)ch * c->hpc * G) * s->head_dim;
            a.q = (const char *)q + head0 * qes;
            a.o = o + head0;
            a.k = kb;
            a.v = vb;
            e = launch_attention(a, compute);
            if (e == hipSuccess) e = hipEventRecord(c->freed[slot], compute);
            if (e == hipSuccess) c->freed_recorded[slot] = true;
        }
    }
    if (e != hipSuccess) return hip_fail(e, "head-wise streaming");
    return ok();
}

int64_t da_stream_length(const da_stream_ctx *c) { return c ? c->len : 0; }

da_status da_stream_set_length(da_stream_ctx *c, int64_t len) {
    if (!c) return fail(DA_E_INVALID, "context is NULL");
    if (len < 1 || len > c->shape.n_ctx)
        return fail(DA_E_INVALID, "length %lld not in [1, %lld]", (long long)len, (long long)c->shape.n_ctx);
    c->len = len;
    return ok();
}

da_status da_stream_append(da_stream_ctx *c, int32_t n_layers, const void *k_new, const void *v_new,
                           void *const *k_host, void *const *v_host, hipStream_t stream) {
    if (!c) return fail(DA_E_INVALID, "context is NULL");
    if (n_layers < 1) return fail(DA_E_INVALID, "n_layers %d < 1", n_layers);
    if (!k_host || !v_host) return fail(DA_E_INVALID, "host pointer arrays are NULL");
    const da_attn_shape *s = &c->shape;
    if (c->len >= s->n_ctx)
        return fail(DA_E_INVALID, "host caches are full (%lld rows)", (long long)s->n_ctx);
    DA_TRY(check_ptr(k_new, "k_new"));
    DA_TRY(check_ptr(v_new, "v_new"));
    const int64_t n_heads = (int64_t)n_layers * s->n_kv_heads;
    if (n_heads > 0x7FFFFFFF) return fail(DA_E_INVALID, "too many layer-heads");
    for (int64_t i = 0; i < n_heads; ++i) {
        DA_TRY(check_pinned(k_host[i], "k_host", i, true));
        DA_TRY(check_pinned(v_host[i], "v_host", i, true));
    }
    // the rows go straight into the host caches, kAppendMaxHeads heads per launch
    const int64_t row = (int64_t)s->head_dim * esize(s->kv_dtype);   // one token of one head
    AppendArgs a;
    a.k_new = (const uint8_t *)k_new;
    a.v_new = (const uint8_t *)v_new;
    a.Hkv = s->n_kv_heads;
    a.batch = s->batch;
    a.row = row;
    a.dst_off = c->len * row;
    a.dst_bstride = s->n_ctx * row;
    hipError_t e = hipSuccess;
    for (int64_t h0 = 0; h0 < n_heads && e == hipSuccess; h0 += kAppendMaxHeads) {
        a.head0 = (int32_t)h0;
        a.n_heads = (int32_t)std::min<int64_t>(kAppendMaxHeads, n_heads - h0);
        for (int i = 0; i < a.n_heads; ++i) {
            a.k_dst[i] = (uint8_t *)k_host[h0 + i];
            a.v_dst[i] = (uint8_t *)v_host[h0 + i];
        }
        e = launch_append(a, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "append");
    c->len += 1;
    return ok();
}

void da_stream_destroy(da_stream_ctx *c) {
    if (!c) return;
    for (int i = 0; i < 2; ++i) {
        (void)hipEventDestroy(c->ready[i]);
        (void)hipEventDestroy(c->freed[i]);
    }
    delete c;
}

}  // extern "C"
