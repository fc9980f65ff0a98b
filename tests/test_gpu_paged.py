"""Page metadata, bound-score top-K selection and sparse attention on the GPU
against the fp64 oracle (TinyServe's query-aware page selection).

Metadata must equal the oracle's by value (min/max are exact).  Selected sets
must equal the oracle's except pages within 1e-5 relative of the oracle's
k-th score.  Sparse attention is checked against the oracle evaluated on the
GPU's own selected set (so a tie decision cannot fail a correct kernel), at
|err| <= 1e-5 on small shapes and 1e-3 at full size, and max|err|/rms <= 1e-4.
"""
import numpy as np
import pytest

import synth
from oracle import bound_scores, decode_attention, page_meta, sparse_attention
from oracle.numerics import as_f64
from gpu_util import assert_close, check_selection, each_row, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,S,N,D", [("f16", 16, 1000, 64), ("bf16", 4, 333, 128),
                                      ("f32", 64, 130, 64), ("f16", 1, 50, 128),
                                      ("f16", 1024, 3000, 64)])
def test_page_meta_exact(da, dt, S, N, D):
    c = synth.paged_case([200, S, N, D], 2, 3, D, N, S, 1, dtype=dt)
    kmin, kmax = da.da_build_page_meta(to_dev(c.k, dt), S)
    rmin, rmax = page_meta(as_f64(c.k, dt), S)
    assert np.array_equal(as_f64(from_dev(kmin, dt), dt), rmin)
    assert np.array_equal(as_f64(from_dev(kmax, dt), dt), rmax)


def run_select(da, c, qdt, kdt, want_scores=True):
    import torch
    q = to_dev(c.q, qdt)
    k = to_dev(c.k, kdt)
    N = c.k.shape[2]
    kmin, kmax = da.da_build_page_meta(k, c.page_size)
    idx, score = da.da_select_pages(q, kmin, kmax, c.page_size, c.top_k, N, want_scores=True)
    torch.cuda.synchronize()
    return q, k, idx.cpu().numpy(), score.cpu().numpy()


SEL_CASES = [
    # B, H, D, N, S, top_k, dtype(q/kv)
    (2, 3, 64, 1000, 16, 5, "f16"),       # partial last page
    (1, 4, 128, 4096, 16, 128, "f16"),
    (2, 2, 64, 777, 4, 37, "f16"),
    (1, 2, 64, 333, 1, 40, "f16"),         # one-token pages: bound = q.k
    (2, 2, 128, 2048, 64, 3, "bf16"),
    (1, 2, 64, 640, 16, 40, "f32"),        # top_k = P: every page
    (32, 8, 64, 1024, 16, 24, "f16"),      # 256 heads, one split each
    (16, 16, 64, 4096, 16, 100, "f16"),    # 256 heads x 4 splits merged in the workgroup
    (1, 2, 64, 3000, 1024, 2, "f16"),      # the largest pages: 3, the last 952 tokens
]


@pytest.mark.parametrize("B,H,D,N,S,K,dt", SEL_CASES)
def test_select_and_sparse_attention(da, B, H, D, N, S, K, dt):
    c = synth.paged_case([201, B, H, D, N, S, K], B, H, D, N, S, K, dtype=dt)
    q, k, idx, score = run_select(da, c, dt, dt)
    q64, k64, v64 = as_f64(c.q, dt), as_f64(c.k, dt), as_f64(c.v, dt)
    rmin, rmax = page_meta(k64, S)
    r = bound_scores(q64, rmin, rmax)
    mag = np.einsum("bhd,bhpd->bhp", np.abs(q64), np.maximum(np.abs(rmin), np.abs(rmax)))
    assert np.all(np.abs(score - r) <= 1e-6 * mag + 1e-30), "bound scores"
    check_selection(idx, r, K)
    if S == 1:
        np.testing.assert_allclose(r, np.einsum("bhd,bhnd->bhn", q64, k64), atol=1e-9)
    o = da.da_decode_attention_paged(q, k, to_dev(c.v, dt), torch_idx(idx), S, scale=c.scale)
    ref = sparse_attention(q64, k64, v64, idx, S, c.scale)
    assert_close(o.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=f"sparse {dt} S{S} K{K}")


@pytest.mark.parametrize("B,H,D,N,S,K,dt", SEL_CASES)
def test_fused_select_and_attention(da, B, H, D, N, S, K, dt):
    """da_decode_attention_sparse (selection and attention in one kernel):
    the kept pages equal da_select_pages' bit for bit (same scores, same
    radix select), and the output matches the oracle's sparse attention over
    that set (tokens past n_ctx in a partial last page skipped)."""
    import torch
    c = synth.paged_case([201, B, H, D, N, S, K], B, H, D, N, S, K, dtype=dt)
    q, k, v = to_dev(c.q, dt), to_dev(c.k, dt), to_dev(c.v, dt)
    kmin, kmax = da.da_build_page_meta(k, S)
    two = da.da_select_pages(q, kmin, kmax, S, K, N)
    o, idx = da.da_decode_attention_sparse(q, kmin, kmax, k, v, S, K, scale=c.scale, want_idx=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    assert np.array_equal(idx, two.cpu().numpy())
    q64, k64, v64 = as_f64(c.q, dt), as_f64(c.k, dt), as_f64(c.v, dt)
    rmin, rmax = page_meta(k64, S)
    check_selection(idx, bound_scores(q64, rmin, rmax), K)
    ref = sparse_attention(q64, k64, v64, idx, S, c.scale)
    assert_close(o.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=f"fused sparse {dt} S{S} K{K}")


def test_fused_without_page_list(da):
    """page_idx may be NULL: the same output as with it."""
    import torch
    c = synth.paged_case([205], 2, 3, 64, 1000, 16, 5, dtype="f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, 16)
    a = da.da_decode_attention_sparse(q, kmin, kmax, k, v, 16, 5)
    b, _ = da.da_decode_attention_sparse(q, kmin, kmax, k, v, 16, 5, want_idx=True)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_workload3_fused_full_size_every_row(da):
    """TinyServe shape in one kernel (as bench.py's step): the kept pages of
    every (batch row, head) equal the two-kernel path's and pass the selection
    rule against the oracle's bound scores; attention of every head against
    the oracle on that set.  The oracle runs one batch row at a time."""
    import torch
    c = synth.workload3()
    S, K = c.page_size, c.top_k
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, S)
    two = da.da_select_pages(q, kmin, kmax, S, K, 32768)
    o, idx = da.da_decode_attention_sparse(q, kmin, kmax, k, v, S, K, want_idx=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    assert np.array_equal(idx, two.cpu().numpy())
    o = o.cpu().numpy()
    del q, k, v, kmin, kmax

    def row(b):
        q64, k64, v64 = (as_f64(x[b:b + 1], "f16") for x in (c.q, c.k, c.v))
        check_selection(idx[b:b + 1], bound_scores(q64, *page_meta(k64, S)), K)
        ref = sparse_attention(q64, k64, v64, idx[b:b + 1], S, c.scale)
        return max(assert_close(o[b:b + 1, h], ref[:, h], atol=1e-3, rel_rms=1e-4, what=f"w3 fused b{b} h{h}", quiet=True)
                   ["max_abs"] for h in range(ref.shape[1]))

    print(f"[parity] w3 fused all 32x16 heads: max |err| {max(each_row(row, c.q.shape[0])):.2e}", flush=True)


def torch_idx(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()


def test_all_pages_equals_dense(da):
    c = synth.paged_case([202], 2, 4, 128, 1500, 16, 94, dtype="f16")
    P = 94
    idx = np.broadcast_to(np.arange(P, dtype=np.int32), (2, 4, P)).copy()
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    o = da.da_decode_attention_paged(q, k, v, torch_idx(idx), 16).cpu().numpy()
    ref = decode_attention(as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16"), c.scale)
    assert_close(o, ref, atol=1e-5, rel_rms=1e-4, what="all pages = dense")


def test_out_of_range_pages_are_skipped(da):
    c = synth.paged_case([203], 1, 2, 64, 100, 16, 4, dtype="f16")   # P = 7, last page 4 tokens
    idx = np.array([[[0, 3, 6, 99]], [[-1, 2, 5, 1000]]], dtype=np.int32).reshape(1, 2, 4)
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    o = da.da_decode_attention_paged(q, k, v, torch_idx(idx), 16).cpu().numpy()
    # the oracle takes the raw lists and skips the same indices itself
    ref = sparse_attention(as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16"), idx, 16, c.scale)
    assert_close(o[:, :1], ref[:, :1], atol=1e-5, what="skip >= P")
    assert_close(o[:, 1:], ref[:, 1:], atol=1e-5, what="skip < 0")


@pytest.mark.parametrize("split", [0, 32, 16])
def test_all_pages_out_of_range_gives_zero(da, split):
    """A list with no page inside the cache attends nothing: the output is
    zero (not 0/0) on all three merge routes -- in the workgroup (one split
    of 512 positions), the small merge kernel (3 splits of 2 pages) and the
    block merge kernel (6 splits of 1 page) -- beside a row with valid pages."""
    c = synth.paged_case([205], 1, 2, 64, 100, 16, 6, dtype="f16")   # P = 7
    idx = np.array([[[-3, 7, 99, 1 << 20, 8, -100]], [[1, 7, 4, -1, 6, 2]]],
                   dtype=np.int32).reshape(1, 2, 6)
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    o = da.da_decode_attention_paged(q, k, v, torch_idx(idx), 16, split_tokens=split).cpu().numpy()
    ref = sparse_attention(as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16"), idx, 16, c.scale)
    assert not np.any(ref[:, 0]) and np.all(o[:, 0] == 0.0), "empty list: output must be zero"
    assert_close(o, ref, atol=1e-5, what=f"empty and valid lists, split {split}")


def test_split_sizes_agree_paged(da):
    c = synth.paged_case([204], 1, 2, 64, 4000, 16, 60, dtype="f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, 16)
    idx = da.da_select_pages(q, kmin, kmax, 16, 60, 4000)
    ref = sparse_attention(as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16"),
                           idx.cpu().numpy(), 16, c.scale)
    for st in (16, 64, 256, 1024):
        o = da.da_decode_attention_paged(q, k, v, idx, 16, split_tokens=st).cpu().numpy()
        assert_close(o, ref, atol=1e-5, rel_rms=1e-4, what=f"paged split {st}")


def test_workload3_full_size_every_row(da):
    """TinyServe shape (B32 H16 D64 N32768 fp16, page 16, top-128) as two
    calls, in the benchmark's launch configuration: the metadata of every
    page equal by value, the selection of every (batch row, head) within the
    rule, and attention of every head against the oracle on the GPU's set."""
    import torch
    c = synth.workload3()
    S, K = c.page_size, c.top_k
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, S)
    idx = da.da_select_pages(q, kmin, kmax, S, K, 32768)
    o = da.da_decode_attention_paged(q, k, v, idx, S)
    torch.cuda.synchronize()
    idx, o = idx.cpu().numpy(), o.cpu().numpy()
    kmin, kmax = kmin.cpu().numpy(), kmax.cpu().numpy()
    del q, k, v

    def row(b):
        q64, k64, v64 = (as_f64(x[b:b + 1], "f16") for x in (c.q, c.k, c.v))
        rmin, rmax = page_meta(k64, S)
        assert np.array_equal(kmin[b:b + 1].astype(np.float64), rmin), f"kmin row {b}"
        assert np.array_equal(kmax[b:b + 1].astype(np.float64), rmax), f"kmax row {b}"
        n_diff = check_selection(idx[b:b + 1], bound_scores(q64, rmin, rmax), K)
        ref = sparse_attention(q64, k64, v64, idx[b:b + 1], S, c.scale)
        err = max(assert_close(o[b:b + 1, h], ref[:, h], atol=1e-3, rel_rms=1e-4, what=f"w3 b{b} h{h}", quiet=True)
                  ["max_abs"] for h in range(ref.shape[1]))
        return err, n_diff

    rs = each_row(row, c.q.shape[0])
    print(f"[parity] w3 all 32x16 heads: max |err| {max(r[0] for r in rs):.2e}, "
          f"{sum(r[1] for r in rs)} pages swapped inside the tie band", flush=True)


@pytest.mark.parametrize("P,K", [(64, 10), (300, 77), (2048, 128)])
def test_selection_with_exact_ties(da, P, K):
    """Pages are copies of four patterns, so bound scores take four values
    and the k-th score is shared by many pages: the lower indices must win,
    exactly as in the oracle (equal scores are equal in fp32 too)."""
    import torch
    rng = np.random.default_rng(P)
    S, D = 4, 64
    pats = rng.standard_normal((4, S, D)).astype(np.float16)
    which = rng.integers(0, 4, size=P)
    k = pats[which].reshape(1, 1, P * S, D)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    kmin, kmax = da.da_build_page_meta(to_dev(k, "f16"), S)
    idx, score = da.da_select_pages(to_dev(q, "f16"), kmin, kmax, S, K, P * S, want_scores=True)
    torch.cuda.synchronize()
    rmin, rmax = page_meta(as_f64(k, "f16"), S)
    r = bound_scores(as_f64(q, "f16"), rmin, rmax)
    s = score.cpu().numpy()
    # identical pages give identical fp32 scores; rank by (-score, index) on them
    order = sorted(range(P), key=lambda j: (-float(s[0, 0, j]), j))
    assert idx.cpu().numpy()[0, 0].tolist() == sorted(order[:K])
    check_selection(idx.cpu().numpy(), r, K)


@pytest.mark.parametrize("B,Hq,Hkv,D,N,S,K", [(2, 8, 2, 64, 1000, 16, 10), (1, 16, 2, 128, 4096, 16, 100),
                                              (2, 4, 1, 64, 777, 4, 37)])
def test_grouped_query_heads(da, B, Hq, Hkv, D, N, S, K):
    """Grouped-query heads: page metadata per KV head; each query head selects
    its own pages over its KV head's metadata (query head j -> KV head j / G)
    and attends over them.  The oracle is the one-KV-head-per-query-head
    definition on K/V repeated G times.  The two-call and one-kernel routes
    keep the same pages."""
    import torch
    G = Hq // Hkv
    c = synth.dense_case([206, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, "f16", "f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, S)
    idx = da.da_select_pages(q, kmin, kmax, S, K, N)
    o2 = da.da_decode_attention_paged(q, k, v, idx, S, scale=c.scale)
    o1, idx1 = da.da_decode_attention_sparse(q, kmin, kmax, k, v, S, K, scale=c.scale, want_idx=True)
    torch.cuda.synchronize()
    idx, idx1 = idx.cpu().numpy(), idx1.cpu().numpy()
    assert np.array_equal(idx, idx1)
    q64 = as_f64(c.q, "f16")
    k64 = np.repeat(as_f64(c.k, "f16"), G, axis=1)
    v64 = np.repeat(as_f64(c.v, "f16"), G, axis=1)
    rmin, rmax = page_meta(k64, S)
    check_selection(idx, bound_scores(q64, rmin, rmax), K)
    ref = sparse_attention(q64, k64, v64, idx, S, c.scale)
    assert_close(o2.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=f"GQA pages two calls G{G}")
    assert_close(o1.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=f"GQA pages one kernel G{G}")


@pytest.mark.parametrize("S,N,K", [(2, 999, 120), (8, 3001, 90), (32, 5000, 40), (128, 20000, 25),
                                   (512, 70000, 7)])
def test_one_kernel_page_sizes(da, S, N, K):
    """The one-kernel page step over page sizes 2..512 with a partial last
    page: the kept pages equal da_select_pages', attention matches the
    oracle on them."""
    import torch
    B, H, D = 1, 3, 64
    c = synth.paged_case([207, S, N, K], B, H, D, N, S, K, dtype="f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, S)
    two = da.da_select_pages(q, kmin, kmax, S, K, N)
    o, idx = da.da_decode_attention_sparse(q, kmin, kmax, k, v, S, K, scale=c.scale, want_idx=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    assert np.array_equal(idx, two.cpu().numpy())
    q64, k64, v64 = as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16")
    rmin, rmax = page_meta(k64, S)
    check_selection(idx, bound_scores(q64, rmin, rmax), K)
    ref = sparse_attention(q64, k64, v64, idx, S, c.scale)
    assert_close(o.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=f"one kernel S{S} N{N} K{K}")
