"""Decode attention over a large KV cache on AMD Instinct MI355X (gfx950).

The computation lives in libda.so (hand-written HIP kernels behind a C ABI,
include/da.h).  This package is the Python binding: the same entry points,
taking torch tensors.

    import sparse_kv_cache_gqa_amd as da
    o = da.da_decode_attention(q, k, v)                  # dense / GQA
    kmin, kmax = da.da_build_page_meta(k, 16)            # page bounding boxes
    idx = da.da_select_pages(q, kmin, kmax, 16, 128, N)  # top-K pages
    o = da.da_decode_attention_paged(q, k, v, idx, 16)   # sparse attention
    o = da.da_decode_attention_sparse(q, kmin, kmax, k, v, 16, 128)  # both in one kernel
    codes, mn, sc = da.da_quantize_kv4(x)                # uint4 groups of 64
    o = da.da_decode_attention_kv4(q, kc, kmn, ksc, vc, vmn, vsc)
    hs = da.HeadwiseStream(...)                          # head-wise streaming
"""
from ._lib import (DA_BF16, DA_E_HIP, DA_E_INVALID, DA_E_NOT_PINNED,  # noqa: F401
                   DA_E_UNSUPPORTED, DA_E_WORKSPACE, DA_F16, DA_F32, DA_OK, DaAttnShape,
                   DaError, LIB_PATH, load)


from .api import (HeadwiseStream, attn_shape, da_build_page_meta,  # noqa: F401,E402
                  da_decode_attention, da_decode_attention_noalloc, da_decode_attention_kv4, da_decode_attention_n_split,
                  da_decode_attention_paged, da_decode_attention_partials, da_merge_partials,
                  da_decode_attention_workspace, da_decode_attention_paged_workspace,
                  da_decode_attention_kv4_workspace,
                  da_dequantize_kv4, da_headwise_buffer_bytes, da_quantize_kv4,
                  da_select_pages, da_select_tokens, da_decode_attention_topk, da_token_keep_count,
                  da_prefill_attention, da_read_stream, da_decode_attention_sparse)
