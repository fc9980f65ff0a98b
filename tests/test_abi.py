"""The C ABI without a GPU: libda.so loads, exports every function declared in
include/da.h, and its host-side argument checks return the documented status
codes before anything is enqueued (the fake device pointers used here are
never dereferenced, and no call here reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

from sparse_kv_cache_gqa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "da.h")

FAKE = ctypes.c_void_p(0x10000)          # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    # DA_ABI_LIB names another build of the same sources to check instead
    # (the host-sanitizer build that tests/test_abi_sanitized.py makes)
    alt = os.environ.get("DA_ABI_LIB")
    if alt:
        return L.load(alt)
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libda.so is not built (run __graft_entry__.build())")
    return L.load()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(da_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES), "binding and header disagree"


def test_version_matches_header(lib):
    src = open(HEADER).read()
    maj, mi, pa = (int(re.search(rf"#define DA_VERSION_{k} (\d+)", src).group(1))
                   for k in ("MAJOR", "MINOR", "PATCH"))
    assert lib.da_version() == (maj << 16) | (mi << 8) | pa


def test_status_strings(lib):
    for code, name in enumerate(["DA_OK", "DA_E_INVALID", "DA_E_UNSUPPORTED", "DA_E_WORKSPACE",
                                 "DA_E_NOT_PINNED", "DA_E_HIP"]):
        assert lib.da_status_string(code).decode() == name


def shape(**kw):
    d = dict(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, n_ctx=32768, scale=128 ** -0.5,
             q_dtype=L.DA_F32, kv_dtype=L.DA_BF16, split_tokens=0)
    d.update(kw)
    return L.DaAttnShape(**d)


def dense(lib, s, q=FAKE, k=FAKE, v=FAKE, o=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.da_decode_attention(ctypes.byref(s) if s is not None else None, q, k, v, o, ws,
                                   ws_bytes, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=30), L.DA_E_INVALID),           # not a multiple of n_kv_heads
    (dict(n_q_heads=24), L.DA_E_UNSUPPORTED),       # G = 3
    (dict(n_q_heads=128), L.DA_E_UNSUPPORTED),      # G = 16
    (dict(n_kv_heads=0), L.DA_E_INVALID),
    (dict(head_dim=96), L.DA_E_UNSUPPORTED),
    (dict(head_dim=0), L.DA_E_INVALID),
    (dict(n_ctx=0), L.DA_E_INVALID),
    (dict(n_ctx=-5), L.DA_E_INVALID),
    (dict(n_ctx=(1 << 34) + 1), L.DA_E_INVALID),     # the split count must fit int32
    (dict(scale=0.0), L.DA_E_INVALID),
    (dict(scale=float("nan")), L.DA_E_INVALID),
    (dict(scale=float("inf")), L.DA_E_INVALID),
    (dict(q_dtype=L.DA_F16), L.DA_E_UNSUPPORTED),   # fp16 q with bf16 KV
    (dict(kv_dtype=7), L.DA_E_INVALID),
    (dict(split_tokens=17), L.DA_E_INVALID),
    (dict(split_tokens=8), L.DA_E_INVALID),
    (dict(split_tokens=1 << 20), L.DA_E_INVALID),
    (dict(batch=-1), L.DA_E_INVALID),
    (dict(batch=20000), L.DA_E_UNSUPPORTED),        # batch * kv heads > 65535
])
def test_dense_shape_checks(lib, kw, code):
    assert dense(lib, shape(**kw)) == code
    assert lib.da_last_error().decode()


def test_dense_pointer_and_workspace_checks(lib):
    s = shape()
    assert dense(lib, None) == L.DA_E_INVALID
    assert dense(lib, s, q=NULL) == L.DA_E_INVALID
    assert dense(lib, s, k=MISALIGNED) == L.DA_E_INVALID
    assert dense(lib, s, o=NULL) == L.DA_E_INVALID
    assert dense(lib, s, ws=NULL) == L.DA_E_INVALID
    need = lib.da_decode_attention_workspace(ctypes.byref(s))
    assert need == 8 * 32 * 16 * 132 * 4          # B*Hq rows x 16 splits of 2048 x (D+4) fp32
    assert dense(lib, s, ws_bytes=need - 1) == L.DA_E_WORKSPACE


def test_empty_batch_is_a_no_op(lib):
    s = shape(batch=0)
    assert dense(lib, s, q=NULL, k=NULL, v=NULL, o=NULL, ws=NULL, ws_bytes=0) == L.DA_OK
    assert lib.da_quantize_kv4(0, 128, NULL, NULL, NULL, NULL, NULL) == L.DA_OK


def test_workspace_depends_on_split_size(lib):
    s1 = shape(split_tokens=1024)
    s2 = shape(split_tokens=256)
    assert lib.da_decode_attention_workspace(ctypes.byref(s1)) == 8 * 32 * 32 * 132 * 4
    assert lib.da_decode_attention_workspace(ctypes.byref(s2)) == 8 * 32 * 128 * 132 * 4
    assert lib.da_decode_attention_workspace(ctypes.byref(shape(head_dim=96))) == 0


def mha(**kw):
    d = dict(batch=32, n_q_heads=16, n_kv_heads=16, head_dim=64, n_ctx=32768, q_dtype=L.DA_F16,
             kv_dtype=L.DA_F16)
    d.update(kw)
    return shape(**d)


def test_page_checks(lib):
    s = mha()
    meta = lambda ps: lib.da_build_page_meta(ctypes.byref(s), ps, FAKE, FAKE, FAKE, NULL)
    assert meta(3) == L.DA_E_INVALID
    assert meta(0) == L.DA_E_INVALID
    assert meta(2048) == L.DA_E_INVALID
    sel = lambda sh, ps, k: lib.da_select_pages(ctypes.byref(sh), ps, k, FAKE, FAKE, FAKE, FAKE,
                                                NULL, NULL)
    assert sel(s, 16, 0) == L.DA_E_INVALID
    assert sel(s, 16, 2049) == L.DA_E_INVALID
    assert sel(mha(n_q_heads=24), 16, 128) == L.DA_E_INVALID         # 24 query heads over 16 KV heads
    assert sel(mha(n_ctx=16 * 8193), 16, 128) == L.DA_E_UNSUPPORTED   # > 8192 pages
    assert lib.da_select_pages(ctypes.byref(s), 16, 128, FAKE, FAKE, FAKE, MISALIGNED, NULL,
                               NULL) == L.DA_E_INVALID
    paged = lambda sh, k, ws_bytes=1 << 40: lib.da_decode_attention_paged(
        ctypes.byref(sh), 16, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, NULL)
    assert paged(s, 0) == L.DA_E_INVALID
    assert paged(mha(n_q_heads=24), 128) == L.DA_E_INVALID
    need = lib.da_decode_attention_paged_workspace(ctypes.byref(s), 16, 128)
    assert need == 32 * 16 * 4 * 68 * 4           # 128 pages of 16 = 2048 positions / 512
    assert paged(s, 128, need - 4) == L.DA_E_WORKSPACE
    # one unit per query head: batch * n_q_heads must fit the grid's second
    # dimension (here 8192 * 16 = 131072 with batch * n_kv_heads = 16384)
    big = mha(batch=8192, n_q_heads=16, n_kv_heads=2)
    assert lib.da_decode_attention_paged_workspace(ctypes.byref(big), 16, 128) == 0
    assert paged(big, 128) == L.DA_E_UNSUPPORTED
    assert b"65535" in lib.da_last_error()
    sp = lambda sh, ps, k, q=FAKE, idx=NULL: lib.da_decode_attention_sparse(
        ctypes.byref(sh), ps, k, q, FAKE, FAKE, FAKE, FAKE, FAKE, idx, NULL)
    assert sp(s, 3, 128) == L.DA_E_INVALID                              # page size
    assert sp(s, 16, 0) == L.DA_E_INVALID
    assert sp(s, 16, 2049) == L.DA_E_INVALID                            # top_k > P
    assert sp(mha(n_q_heads=24), 16, 128) == L.DA_E_INVALID            # not a multiple of n_kv_heads
    assert sp(mha(n_ctx=16 * 8193), 16, 128) == L.DA_E_UNSUPPORTED      # > 8192 pages
    assert sp(s, 16, 500) == L.DA_E_UNSUPPORTED      # 2048 + 500 + 2 * 8000 + 16 * 64 > 16384
    assert sp(s, 16, 128, q=MISALIGNED) == L.DA_E_INVALID
    assert sp(s, 16, 128, idx=MISALIGNED) == L.DA_E_INVALID
    assert sp(mha(batch=0), 16, 128) == L.DA_OK


def test_token_selection_checks(lib):
    s = mha(n_ctx=1024)
    sel = lambda sh, k, score=NULL: lib.da_select_tokens(ctypes.byref(sh), k, FAKE, FAKE, FAKE, score, NULL)
    assert sel(s, 0) == L.DA_E_INVALID
    assert sel(s, 1025) == L.DA_E_INVALID
    assert sel(mha(n_q_heads=24, n_ctx=1024), 100) == L.DA_E_INVALID       # not a multiple of n_kv_heads
    assert sel(mha(n_ctx=8193), 100) == L.DA_E_UNSUPPORTED                  # > 8192 tokens
    assert sel(s, 100, MISALIGNED) == L.DA_E_INVALID
    assert lib.da_select_tokens(ctypes.byref(s), 100, FAKE, NULL, FAKE, NULL, NULL) == L.DA_E_INVALID
    assert lib.da_select_tokens(ctypes.byref(mha(batch=0, n_ctx=1024)), 5, NULL, NULL, NULL, NULL,
                                NULL) == L.DA_OK


def test_topk_attention_checks(lib):
    s = mha(n_ctx=1024, head_dim=128)
    att = lambda sh, k, idx=NULL: lib.da_decode_attention_topk(ctypes.byref(sh), k, FAKE, FAKE, FAKE, FAKE,
                                                               idx, NULL)
    assert att(s, 0) == L.DA_E_INVALID
    assert att(s, 1025) == L.DA_E_INVALID
    assert att(mha(n_q_heads=24, n_ctx=1024), 100) == L.DA_E_INVALID        # not a multiple of n_kv_heads
    assert att(mha(n_ctx=8192, head_dim=128), 3585) == L.DA_E_UNSUPPORTED    # LDS budget
    assert att(s, 100, MISALIGNED) == L.DA_E_INVALID
    assert lib.da_decode_attention_topk(ctypes.byref(s), 100, FAKE, FAKE, NULL, FAKE, NULL,
                                        NULL) == L.DA_E_INVALID


def test_prefill_checks(lib):
    s = shape(batch=1, n_ctx=4096, q_dtype=L.DA_BF16, kv_dtype=L.DA_BF16)
    pre = lambda sh, c: lib.da_prefill_attention(ctypes.byref(sh), c, FAKE, FAKE, FAKE, FAKE, NULL)
    assert pre(s, 0) == L.DA_E_INVALID
    assert pre(s, 4097) == L.DA_E_INVALID
    assert pre(shape(batch=1, n_ctx=4096), 128) == L.DA_E_UNSUPPORTED                 # fp32 q
    assert pre(shape(batch=1, n_ctx=4096, q_dtype=L.DA_F16, kv_dtype=L.DA_BF16), 128) == L.DA_E_UNSUPPORTED
    assert lib.da_prefill_attention(ctypes.byref(s), 128, FAKE, FAKE, FAKE, NULL, NULL) == L.DA_E_INVALID


def test_kv4_checks(lib):
    q = lambda **kw: lib.da_quantize_kv4(kw.get("n", 4), kw.get("r", 128), FAKE, FAKE, FAKE, FAKE,
                                          NULL)
    assert q(r=96) == L.DA_E_INVALID
    assert q(r=0) == L.DA_E_INVALID
    assert q(n=-1) == L.DA_E_INVALID
    assert lib.da_quantize_kv4(4, 128, MISALIGNED, FAKE, FAKE, FAKE, NULL) == L.DA_E_INVALID
    assert lib.da_dequantize_kv4(4, 100, FAKE, FAKE, FAKE, FAKE, NULL) == L.DA_E_INVALID
    s = shape(batch=64, n_q_heads=56, n_kv_heads=56, head_dim=128, n_ctx=1024, q_dtype=L.DA_F16)
    att = lambda sh: lib.da_decode_attention_kv4(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE,
                                                 FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL)
    s64 = shape(batch=64, n_q_heads=56, n_kv_heads=56, head_dim=64, n_ctx=1024, q_dtype=L.DA_F16)
    assert att(s64) == L.DA_E_UNSUPPORTED
    sbf = shape(batch=64, n_q_heads=56, n_kv_heads=56, head_dim=128, n_ctx=1024, q_dtype=L.DA_BF16)
    assert att(sbf) == L.DA_E_UNSUPPORTED
    # default uint4 split: the longest power of two from 256 tokens that keeps
    # >= 2048 waves -- one 1024-token split per head at B64 H56, 256-token
    # splits for a single row of 4 heads, 2048 (two per head) for 1024 units
    # at 4096 tokens
    ws = lambda **kw: lib.da_decode_attention_kv4_workspace(ctypes.byref(shape(
        head_dim=128, q_dtype=L.DA_F16, **kw)))
    assert lib.da_decode_attention_kv4_workspace(ctypes.byref(s)) == 64 * 56 * 1 * 132 * 4
    assert ws(batch=1, n_q_heads=4, n_kv_heads=4, n_ctx=1024) == 4 * 4 * 132 * 4
    assert ws(batch=16, n_q_heads=64, n_kv_heads=64, n_ctx=4096) == 1024 * 2 * 132 * 4
    assert ws(batch=16, n_q_heads=64, n_kv_heads=64, n_ctx=4096, split_tokens=1024) == 1024 * 4 * 132 * 4


def test_read_stream_checks(lib):
    r = lambda buf=FAKE, nb=1 << 20, g=16, sink=FAKE: lib.da_read_stream(buf, nb, g, sink, NULL)
    assert r(nb=0) == L.DA_E_INVALID
    assert r(nb=1000) == L.DA_E_INVALID                 # not a multiple of 16
    assert r(nb=(1 << 40) + 16) == L.DA_E_INVALID
    assert r(g=0) == L.DA_E_INVALID
    assert r(g=65536) == L.DA_E_INVALID
    assert r(nb=160, g=11) == L.DA_E_INVALID            # more groups than 16-byte units
    assert r(buf=NULL) == L.DA_E_INVALID
    assert r(buf=MISALIGNED) == L.DA_E_INVALID
    assert r(sink=NULL) == L.DA_E_INVALID


def test_headwise_sizes_match_the_pages_and_checks(lib):
    # Llama-3-8B, 1M tokens, bf16: one head's K+V is 512 MiB; a layer is 4 GiB
    s = shape(batch=1, n_ctx=1 << 20)
    assert lib.da_headwise_buffer_bytes(ctypes.byref(s), 1) == 512 << 20
    assert 2 * lib.da_headwise_buffer_bytes(ctypes.byref(s), 1) == 1 << 30     # "1 GB" on GPU
    assert 2 * lib.da_headwise_buffer_bytes(ctypes.byref(s), 8) == 8 << 30     # layer-wise "8 GB"
    assert lib.da_headwise_buffer_bytes(ctypes.byref(s), 3) == 0
    ctx = ctypes.c_void_p()
    assert lib.da_stream_create(ctypes.byref(s), 3, ctypes.byref(ctx)) == L.DA_E_INVALID
    assert lib.da_stream_create(ctypes.byref(s), 16, ctypes.byref(ctx)) == L.DA_E_INVALID
    assert lib.da_stream_create(ctypes.byref(s), 1, None) == L.DA_E_INVALID
    arr = (ctypes.c_void_p * 1)(FAKE)
    assert lib.da_stream_headwise(None, 1, arr, arr, FAKE, FAKE, FAKE, FAKE, FAKE, 1, NULL,
                                  ctypes.c_void_p(1)) == L.DA_E_INVALID
    assert lib.da_stream_length(None) == 0
    assert lib.da_stream_set_length(None, 5) == L.DA_E_INVALID
    assert lib.da_stream_append(None, 1, FAKE, FAKE, arr, arr, NULL) == L.DA_E_INVALID
    assert lib.da_stream_buffer_bytes(None) == 0
    assert lib.da_stream_workspace(None) == 0
    lib.da_stream_destroy(None)


def test_token_keep_count_matches_the_oracle(lib):
    """FlexGen's kept-token count (ceil of 10% of the context) as the library
    computes it, against the oracle's rule, for every context 1..20000."""
    from oracle import keep_count
    for n in range(1, 20001):
        assert lib.da_token_keep_count(n) == keep_count(n), n
    assert lib.da_token_keep_count(1024) == 103
    assert lib.da_token_keep_count(0) == 0
    assert lib.da_token_keep_count(-3) == 0
    assert lib.da_token_keep_count(1 << 40) == -(-(1 << 40) // 10)


def test_noalloc_checks(lib):
    """The allocation-free entry point refuses, before anything is enqueued,
    a shape whose split-K partials exceed its fixed scratch array, as well as
    the usual bad arguments."""
    assert lib.da_decode_attention_noalloc_max_scratch() == 16 << 20
    call = lambda s, q=FAKE, o=FAKE: lib.da_decode_attention_noalloc(ctypes.byref(s), q, FAKE, FAKE, o, NULL)
    big = shape(batch=64, n_ctx=1 << 20)          # 64 x 32 rows x 512 splits x 132 floats
    assert lib.da_decode_attention_workspace(ctypes.byref(big)) > (16 << 20)
    assert call(big) == L.DA_E_UNSUPPORTED
    assert b"scratch" in lib.da_last_error()
    assert call(shape(head_dim=96)) == L.DA_E_UNSUPPORTED
    assert call(shape(), q=MISALIGNED) == L.DA_E_INVALID
    assert call(shape(), o=NULL) == L.DA_E_INVALID
    assert call(shape(batch=0)) == L.DA_OK
