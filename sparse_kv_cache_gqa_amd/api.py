"""Python binding of libda.so: the same entry points, taking torch tensors.

Argument marshalling only: shapes and dtypes are read from the tensors, the
output and the workspace are allocated with torch (device memory plumbing),
and the raw pointers plus the current HIP stream go to the C ABI.  Every step
of the computation runs in the library's kernels; if libda.so is missing the
calls raise.
"""
from __future__ import annotations

import contextlib
import ctypes
import math

import torch

from ._lib import (DA_BF16, DA_F16, DA_F32, DaAttnShape, check, load)

_DT = {torch.float32: DA_F32, torch.float16: DA_F16, torch.bfloat16: DA_BF16}


def _vp(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous GPU tensors")


def attn_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, scale=None, q_dtype=DA_F32,
               kv_dtype=DA_BF16, split_tokens=0) -> DaAttnShape:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DaAttnShape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, scale, q_dtype, kv_dtype,
                       split_tokens)


def _dense_shape(q, k, scale, split_tokens, kv_dtype=None):
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B][Hq][D] and k [B][Hkv][N][D]")
    B, Hq, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    if Bk != B or (kv_dtype is None and Dk != D):
        raise ValueError("q and k disagree on batch or head_dim")
    kvd = _DT[k.dtype] if kv_dtype is None else kv_dtype
    return attn_shape(B, Hq, Hkv, D, N, scale, _DT[q.dtype], kvd, split_tokens)


def _expect(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _on(stream):
    """Context for allocating the temporaries of a call that runs on `stream`:
    the caching allocator then orders their reuse after the call's kernels
    (a block freed on one stream is reused only by work on that stream)."""
    if stream is None:
        return contextlib.nullcontext()
    if not hasattr(stream, "cuda_stream"):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _new(stream, shape, dtype, device):
    """torch.empty allocated for use on `stream` (see _on)."""
    with _on(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _ws(nbytes: int, device, stream):
    return _new(stream, max(int(nbytes), 16), torch.uint8, device)


# ---------------------------------------------------------------------------
def da_decode_attention(q, k, v, scale=None, split_tokens=0, out=None, ws=None, stream=None):
    """o[b, j] = softmax(scale q[b,j] . K[b, j//G]^T) V[b, j//G]; fp32 [B][Hq][D]."""
    lib = load()
    _dev(q, k, v, out, ws)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    s = _dense_shape(q, k, scale, split_tokens)
    need = lib.da_decode_attention_workspace(ctypes.byref(s))
    _expect(out, q.shape, torch.float32, "out")
    if out is None:
        out = _new(stream, q.shape, torch.float32, q.device)
    if ws is None:
        ws = _ws(need, q.device, stream)
    check(lib.da_decode_attention(ctypes.byref(s), _vp(q), _vp(k), _vp(v), _vp(out), _vp(ws),
                                  _nbytes(ws), _stream(stream)))
    return out


def da_decode_attention_noalloc(q, k, v, out, scale=None, split_tokens=0, stream=None):
    """da_decode_attention with the split-K partials in the library's fixed
    per-GPU scratch array: no workspace, and `out` (fp32 [B][Hq][D]) is the
    caller's, so the call allocates nothing."""
    lib = load()
    _dev(q, k, v, out)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    s = _dense_shape(q, k, scale, split_tokens)
    _expect(out, q.shape, torch.float32, "out")
    check(lib.da_decode_attention_noalloc(ctypes.byref(s), _vp(q), _vp(k), _vp(v), _vp(out),
                                          _stream(stream)))
    return out


def da_decode_attention_workspace(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, q_dtype=DA_F32,
                                  kv_dtype=DA_BF16, split_tokens=0) -> int:
    s = attn_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, None, q_dtype, kv_dtype,
                   split_tokens)
    return int(load().da_decode_attention_workspace(ctypes.byref(s)))


def da_decode_attention_paged_workspace(batch, n_heads, head_dim, n_ctx, page_size, top_k,
                                        q_dtype=DA_F16, kv_dtype=DA_F16, split_tokens=0) -> int:
    s = attn_shape(batch, n_heads, n_heads, head_dim, n_ctx, None, q_dtype, kv_dtype, split_tokens)
    return int(load().da_decode_attention_paged_workspace(ctypes.byref(s), page_size, top_k))


def da_decode_attention_kv4_workspace(batch, n_q_heads, n_kv_heads, head_dim, n_ctx,
                                      q_dtype=DA_F16, split_tokens=0) -> int:
    s = attn_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, None, q_dtype, DA_F16,
                   split_tokens)
    return int(load().da_decode_attention_kv4_workspace(ctypes.byref(s)))


def da_decode_attention_n_split(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, split_tokens=0) -> int:
    s = attn_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, None, DA_F32, DA_BF16, split_tokens)
    return int(load().da_decode_attention_n_split(ctypes.byref(s)))


def da_decode_attention_partials(q, k, v, scale=None, split_tokens=0, ws=None, stream=None):
    """Split-K pass only: fp32 partials [B][Hq][n_split][D+4] = (u[D], m, l, pad, pad)."""
    lib = load()
    _dev(q, k, v, ws)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    s = _dense_shape(q, k, scale, split_tokens)
    ns = int(lib.da_decode_attention_n_split(ctypes.byref(s)))
    shape = (q.shape[0], q.shape[1], ns, q.shape[2] + 4)
    _expect(ws, shape, torch.float32, "ws")
    if ws is None:
        ws = _new(stream, shape, torch.float32, q.device)
    check(lib.da_decode_attention_partials(ctypes.byref(s), _vp(q), _vp(k), _vp(v), _vp(ws),
                                           _nbytes(ws), _stream(stream)))
    return ws


def da_read_stream(buf, n_groups=4096, sink=None, stream=None):
    """Measurement aid: read every byte of the device tensor `buf` once
    (non-temporal, n_groups contiguous chunks); returns sink [n_groups] uint32,
    the XOR of each chunk's 32-bit words."""
    lib = load()
    _dev(buf, sink)
    nb = _nbytes(buf)
    if sink is None:
        sink = _new(stream, n_groups, torch.int32, buf.device)
    _expect(sink, (n_groups,), torch.int32, "sink")
    check(lib.da_read_stream(_vp(buf), nb, n_groups, _vp(sink), _stream(stream)))
    return sink


def da_merge_partials(partials, out=None, stream=None):
    """partials [..., n_split, D+4] fp32 -> o [..., D] fp32."""
    lib = load()
    _dev(partials, out)
    if partials.dtype != torch.float32:
        raise ValueError("partials must be float32")
    ns, D = partials.shape[-2], partials.shape[-1] - 4
    lead = tuple(partials.shape[:-2])
    rows = partials.numel() // (ns * (D + 4))
    _expect(out, lead + (D,), torch.float32, "out")
    if out is None:
        out = _new(stream, lead + (D,), torch.float32, partials.device)
    check(lib.da_merge_partials(rows, ns, D, _vp(partials), _vp(out), _stream(stream)))
    return out


def da_build_page_meta(k, page_size, kmin=None, kmax=None, stream=None):
    """Per-page per-channel key min and max: ([B][H][P][D], [B][H][P][D])."""
    lib = load()
    _dev(k, kmin, kmax)
    B, H, N, D = k.shape
    P = -(-N // page_size)
    s = attn_shape(B, H, H, D, N, None, _DT[k.dtype], _DT[k.dtype])
    _expect(kmin, (B, H, P, D), k.dtype, "kmin")
    _expect(kmax, (B, H, P, D), k.dtype, "kmax")
    if kmin is None:
        kmin = _new(stream, (B, H, P, D), k.dtype, k.device)
    if kmax is None:
        kmax = _new(stream, (B, H, P, D), k.dtype, k.device)
    check(lib.da_build_page_meta(ctypes.byref(s), page_size, _vp(k), _vp(kmin), _vp(kmax),
                                 _stream(stream)))
    return kmin, kmax


def da_select_pages(q, kmin, kmax, page_size, top_k, n_ctx, page_idx=None, page_score=None,
                    want_scores=False, stream=None):
    """Top-k pages by the bound score per (b, query head), ascending int32
    [B][Hq][top_k]; kmin/kmax [B][Hkv][P][D] (query head j reads KV head
    j / (Hq / Hkv))."""
    lib = load()
    _dev(q, kmin, kmax, page_idx, page_score)
    B, H, D = q.shape
    Hkv = kmin.shape[1]
    P = -(-n_ctx // page_size)
    _expect(kmin, (B, Hkv, P, D), kmin.dtype, "kmin")
    _expect(kmax, (B, Hkv, P, D), kmin.dtype, "kmax")
    _expect(page_idx, (B, H, top_k), torch.int32, "page_idx")
    _expect(page_score, (B, H, P), torch.float32, "page_score")
    s = attn_shape(B, H, Hkv, D, n_ctx, None, _DT[q.dtype], _DT[kmin.dtype])
    if page_idx is None:
        page_idx = _new(stream, (B, H, top_k), torch.int32, q.device)
    if want_scores and page_score is None:
        page_score = _new(stream, (B, H, P), torch.float32, q.device)
    check(lib.da_select_pages(ctypes.byref(s), page_size, top_k, _vp(q), _vp(kmin), _vp(kmax),
                              _vp(page_idx), _vp(page_score), _stream(stream)))
    return (page_idx, page_score) if want_scores else page_idx


def da_select_tokens(q, k, top_k, token_idx=None, token_score=None, want_scores=False, stream=None):
    """Top-k tokens by exact score q . k per (b, query head), ascending int32
    [B][Hq][top_k]; k [B][Hkv][N][D] (query head j reads KV head j / (Hq / Hkv))."""
    lib = load()
    _dev(q, k, token_idx, token_score)
    B, H, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    _expect(k, (B, Hkv, N, D), k.dtype, "k")
    _expect(token_idx, (B, H, top_k), torch.int32, "token_idx")
    _expect(token_score, (B, H, N), torch.float32, "token_score")
    s = attn_shape(B, H, Hkv, D, N, None, _DT[q.dtype], _DT[k.dtype])
    if token_idx is None:
        token_idx = _new(stream, (B, H, top_k), torch.int32, q.device)
    if want_scores and token_score is None:
        token_score = _new(stream, (B, H, N), torch.float32, q.device)
    check(lib.da_select_tokens(ctypes.byref(s), top_k, _vp(q), _vp(k), _vp(token_idx),
                               _vp(token_score), _stream(stream)))
    return (token_idx, token_score) if want_scores else token_idx


def da_token_keep_count(n_ctx) -> int:
    """Tokens FlexGen's top-10% sparse attention keeps per query (computed by
    the library: ceil(n_ctx / 10)); 0 if n_ctx < 1."""
    return int(load().da_token_keep_count(int(n_ctx)))


def da_decode_attention_topk(q, k, v, top_k, scale=None, token_idx=None, want_idx=False, out=None,
                             stream=None):
    """FlexGen's token-level sparse attention in one kernel: the top_k tokens
    by exact score, then attention over them only; fp32 [B][H][D]."""
    lib = load()
    _dev(q, k, v, token_idx, out)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    B, H, D = q.shape
    s = _dense_shape(q, k, scale, 0)
    _expect(out, q.shape, torch.float32, "out")
    _expect(token_idx, (B, H, top_k), torch.int32, "token_idx")
    if out is None:
        out = _new(stream, q.shape, torch.float32, q.device)
    if want_idx and token_idx is None:
        token_idx = _new(stream, (B, H, top_k), torch.int32, q.device)
    check(lib.da_decode_attention_topk(ctypes.byref(s), top_k, _vp(q), _vp(k), _vp(v), _vp(out),
                                       _vp(token_idx), _stream(stream)))
    return (out, token_idx) if want_idx else out


def da_prefill_attention(q, k, v, scale=None, out=None, stream=None):
    """Chunked prefill: q [B][Hq][C][D] at the last C positions of k, v
    [B][Hkv][T][D] (causal); fp32 [B][Hq][C][D]."""
    lib = load()
    _dev(q, k, v, out)
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("q, k and v must share a dtype; k and v a shape")
    B, Hq, C, D = q.shape
    Bk, Hkv, T, Dk = k.shape
    if (Bk, Dk) != (B, D) or C > T:
        raise ValueError("q [B][Hq][C][D] needs k, v [B][Hkv][T][D] with T >= C")
    s = attn_shape(B, Hq, Hkv, D, T, scale, _DT[q.dtype], _DT[k.dtype])
    _expect(out, q.shape, torch.float32, "out")
    if out is None:
        out = _new(stream, q.shape, torch.float32, q.device)
    check(lib.da_prefill_attention(ctypes.byref(s), C, _vp(q), _vp(k), _vp(v), _vp(out), _stream(stream)))
    return out


def da_decode_attention_paged(q, k, v, page_idx, page_size, scale=None, split_tokens=0, out=None,
                              ws=None, stream=None):
    """Attention over the tokens of the listed pages only; fp32 [B][H][D]."""
    lib = load()
    _dev(q, k, v, page_idx, out, ws)
    s = _dense_shape(q, k, scale, split_tokens)
    top_k = page_idx.shape[-1]
    _expect(page_idx, (q.shape[0], q.shape[1], top_k), torch.int32, "page_idx")
    _expect(out, q.shape, torch.float32, "out")
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    need = lib.da_decode_attention_paged_workspace(ctypes.byref(s), page_size, top_k)
    if out is None:
        out = _new(stream, q.shape, torch.float32, q.device)
    if ws is None:
        ws = _ws(need, q.device, stream)
    check(lib.da_decode_attention_paged(ctypes.byref(s), page_size, top_k, _vp(page_idx), _vp(q),
                                        _vp(k), _vp(v), _vp(out), _vp(ws), _nbytes(ws),
                                        _stream(stream)))
    return out


def da_decode_attention_sparse(q, kmin, kmax, k, v, page_size, top_k, scale=None, out=None,
                               page_idx=None, want_idx=False, stream=None):
    """Page selection and attention over the kept pages in one kernel
    (TinyServe's decode step); fp32 [B][H][D], and the kept pages
    [B][H][top_k] int32 when want_idx (or page_idx) is given."""
    lib = load()
    _dev(q, kmin, kmax, k, v, out, page_idx)
    s = _dense_shape(q, k, scale, 0)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    B, H, N, D = k.shape
    P = -(-N // page_size)
    _expect(kmin, (B, H, P, D), k.dtype, "kmin")
    _expect(kmax, (B, H, P, D), k.dtype, "kmax")
    _expect(out, q.shape, torch.float32, "out")
    _expect(page_idx, (q.shape[0], q.shape[1], top_k), torch.int32, "page_idx")
    if out is None:
        out = _new(stream, q.shape, torch.float32, q.device)
    if page_idx is None and want_idx:
        page_idx = _new(stream, (q.shape[0], q.shape[1], top_k), torch.int32, q.device)
    check(lib.da_decode_attention_sparse(ctypes.byref(s), page_size, top_k, _vp(q), _vp(kmin), _vp(kmax),
                                         _vp(k), _vp(v), _vp(out), _vp(page_idx), _stream(stream)))
    return (out, page_idx) if (want_idx or page_idx is not None) else out


def da_quantize_kv4(x, codes=None, gmin=None, gscale=None, stream=None):
    """fp16 [..., R] -> (codes uint8 [..., R/2], min fp16 [..., R/64], scale fp16 [..., R/64])."""
    lib = load()
    _dev(x, codes, gmin, gscale)
    if x.dtype != torch.float16:
        raise ValueError("x must be float16")
    R = x.shape[-1]
    lead = tuple(x.shape[:-1])
    n_rows = x.numel() // R if R else 0
    _expect(codes, lead + (R // 2,), torch.uint8, "codes")
    _expect(gmin, lead + (R // 64,), torch.float16, "gmin")
    _expect(gscale, lead + (R // 64,), torch.float16, "gscale")
    if codes is None:
        codes = _new(stream, lead + (R // 2,), torch.uint8, x.device)
    if gmin is None:
        gmin = _new(stream, lead + (R // 64,), torch.float16, x.device)
    if gscale is None:
        gscale = _new(stream, lead + (R // 64,), torch.float16, x.device)
    check(lib.da_quantize_kv4(n_rows, R, _vp(x), _vp(codes), _vp(gmin), _vp(gscale),
                              _stream(stream)))
    return codes, gmin, gscale


def da_dequantize_kv4(codes, gmin, gscale, out=None, stream=None):
    """(codes, min, scale) -> fp16 fp16(min + code * scale)."""
    lib = load()
    _dev(codes, gmin, gscale, out)
    R = codes.shape[-1] * 2
    lead = tuple(codes.shape[:-1])
    n_rows = codes.numel() * 2 // R if R else 0
    if codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    _expect(gmin, lead + (R // 64,), torch.float16, "gmin")
    _expect(gscale, lead + (R // 64,), torch.float16, "gscale")
    _expect(out, lead + (R,), torch.float16, "out")
    if out is None:
        out = _new(stream, lead + (R,), torch.float16, codes.device)
    check(lib.da_dequantize_kv4(n_rows, R, _vp(codes), _vp(gmin), _vp(gscale), _vp(out),
                                _stream(stream)))
    return out


def da_decode_attention_kv4(q, k_codes, k_min, k_scale, v_codes, v_min, v_scale, scale=None,
                            split_tokens=0, out=None, ws=None, stream=None):
    """Decode attention over a uint4 cache; fp32 [B][Hq][D]."""
    lib = load()
    _dev(q, k_codes, k_min, k_scale, v_codes, v_min, v_scale, out, ws)
    B, Hq, D = q.shape
    if k_codes.dim() != 4 or k_codes.shape[-1] * 2 != D:
        raise ValueError("codes must be [B][Hkv][N][D/2]")
    Hkv, N = k_codes.shape[1], k_codes.shape[2]
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _expect(t, (B, Hkv, N, D // 2), torch.uint8, name)
    for t, name in ((k_min, "k_min"), (k_scale, "k_scale"), (v_min, "v_min"), (v_scale, "v_scale")):
        _expect(t, (B, Hkv, N, D // 64), torch.float16, name)
    _expect(out, q.shape, torch.float32, "out")
    s = attn_shape(B, Hq, Hkv, D, N, scale, _DT[q.dtype], DA_F16, split_tokens)
    need = lib.da_decode_attention_kv4_workspace(ctypes.byref(s))
    if out is None:
        out = _new(stream, q.shape, torch.float32, q.device)
    if ws is None:
        ws = _ws(need, q.device, stream)
    check(lib.da_decode_attention_kv4(ctypes.byref(s), _vp(q), _vp(k_codes), _vp(k_min),
                                      _vp(k_scale), _vp(v_codes), _vp(v_min), _vp(v_scale),
                                      _vp(out), _vp(ws), _nbytes(ws), _stream(stream)))
    return out


def da_headwise_buffer_bytes(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, kv_dtype=DA_BF16,
                             q_dtype=DA_F32, heads_per_chunk=1) -> int:
    s = attn_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, None, q_dtype, kv_dtype)
    return int(load().da_headwise_buffer_bytes(ctypes.byref(s), heads_per_chunk))


class HeadwiseStream:
    """da_stream_* context: head-wise streamed decode over pinned host KV."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, n_ctx, q_dtype=DA_F32,
                 kv_dtype=DA_BF16, heads_per_chunk=1, scale=None, split_tokens=0):
        self._lib = load()
        self.shape = attn_shape(batch, n_q_heads, n_kv_heads, head_dim, n_ctx, scale, q_dtype,
                                kv_dtype, split_tokens)
        self.heads_per_chunk = heads_per_chunk
        self._ctx = ctypes.c_void_p()
        check(self._lib.da_stream_create(ctypes.byref(self.shape), heads_per_chunk,
                                         ctypes.byref(self._ctx)))

    @staticmethod
    def _check_dtype(t, want, name):
        if _DT.get(t.dtype) != want:
            raise ValueError(f"{name}: dtype {t.dtype} does not match the context's")

    @property
    def buffer_bytes(self) -> int:
        return int(self._lib.da_stream_buffer_bytes(self._ctx))

    @property
    def workspace_bytes(self) -> int:
        return int(self._lib.da_stream_workspace(self._ctx))

    def da_stream_headwise(self, k_host, v_host, buf0, buf1, q, out, ws, compute, copy):
        """k_host/v_host: lists (layer-major) of pinned host tensors [B][N][D]."""
        _dev(buf0, buf1, q, out, ws)
        n = len(k_host)
        if n % self.shape.n_kv_heads or len(v_host) != n:
            raise ValueError("need n_layers * n_kv_heads host tensors for K and for V")
        for t in list(k_host) + list(v_host):
            if t.is_cuda or not t.is_contiguous():
                raise ValueError("host KV tensors must be contiguous CPU tensors")
        hb = self.buffer_bytes // (2 * self.heads_per_chunk)
        for t in list(k_host) + list(v_host):
            if t.numel() * t.element_size() != hb:
                raise ValueError(f"each host head must hold {hb} bytes")
        for b in (buf0, buf1):
            if b.numel() * b.element_size() < self.buffer_bytes:
                raise ValueError(f"ping-pong buffers need {self.buffer_bytes} bytes")
        L = n // self.shape.n_kv_heads
        qshape = (L, self.shape.batch, self.shape.n_q_heads, self.shape.head_dim)
        if tuple(q.shape) != qshape or tuple(out.shape) != qshape or out.dtype != torch.float32:
            raise ValueError(f"q and out must be {qshape} (out fp32)")
        self._check_dtype(q, self.shape.q_dtype, "q")
        for t in list(k_host) + list(v_host):
            self._check_dtype(t, self.shape.kv_dtype, "host KV")
        kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_host])
        vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_host])
        check(self._lib.da_stream_headwise(self._ctx, n // self.shape.n_kv_heads, kp, vp,
                                           _vp(buf0), _vp(buf1), _vp(q), _vp(out), _vp(ws),
                                           _nbytes(ws), _stream(compute), _stream(copy)))
        return out

    @property
    def length(self) -> int:
        """Rows attended per batch row (the host caches hold n_ctx rows)."""
        return int(self._lib.da_stream_length(self._ctx))

    def set_length(self, n):
        check(self._lib.da_stream_set_length(self._ctx, int(n)))

    def append(self, k_new, v_new, k_host, v_host, stream=None):
        """Copy the new token's rows k_new, v_new [L][B][Hkv][D] (device) into
        row `length` of every host cache, then extend the length by one."""
        _dev(k_new, v_new)
        n = len(k_host)
        if n % self.shape.n_kv_heads or len(v_host) != n:
            raise ValueError("need n_layers * n_kv_heads host tensors for K and for V")
        L = n // self.shape.n_kv_heads
        want = (L, self.shape.batch, self.shape.n_kv_heads, self.shape.head_dim)
        for t in (k_new, v_new):
            if tuple(t.shape) != want or not t.is_contiguous():
                raise ValueError(f"new rows must be contiguous {want}")
            self._check_dtype(t, self.shape.kv_dtype, "new rows")
        for t in list(k_host) + list(v_host):
            if t.is_cuda or not t.is_contiguous():
                raise ValueError("host KV tensors must be contiguous CPU tensors")
            self._check_dtype(t, self.shape.kv_dtype, "host KV")
        kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_host])
        vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_host])
        check(self._lib.da_stream_append(self._ctx, L, _vp(k_new), _vp(v_new), kp, vp, _stream(stream)))

    def close(self):
        if self._ctx:
            self._lib.da_stream_destroy(self._ctx)
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
