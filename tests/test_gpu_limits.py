"""Entry points at the largest sizes their one-workgroup-per-head kernels
accept (the scores of a head live in LDS): page selection at 8192 pages, the
one-kernel page step at its LDS budget of P + K + 2 K S + 16 head_dim =
16384 floats, and the one-kernel top-k attention at its LDS budget of
n_ctx + 2 top_k + 8 head_dim = 16384 floats.  Same bars as the other tests: selected sets equal
the oracle's except near-ties within 1e-5 of the k-th score; attention
against the oracle on the GPU's own set at 1e-3 absolute (1e-5 on the small
top-k shapes) and max|err|/rms <= 1e-4."""
import numpy as np
import pytest

import synth
from oracle import bound_scores, decode_attention, keep_count, page_meta, sparse_attention, token_scores
from oracle.numerics import as_f64
from gpu_util import assert_close, check_selection, to_dev

pytestmark = pytest.mark.gpu

MAX_PAGES = 8192
TOPK_LDS_FLOATS = 16384


@pytest.mark.parametrize("K", [500, MAX_PAGES])
def test_select_pages_at_the_page_limit(da, K):
    """8192 pages of 16 tokens (131072 tokens per head); K = all pages is
    dense attention."""
    import torch
    B, H, D, S = 1, 2, 64, 16
    N = MAX_PAGES * S
    c = synth.paged_case([210, K], B, H, D, N, S, K, dtype="f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, S)
    idx = da.da_select_pages(q, kmin, kmax, S, K, N)
    o = da.da_decode_attention_paged(q, k, v, idx, S, scale=c.scale)
    torch.cuda.synchronize()
    idx, o = idx.cpu().numpy(), o.cpu().numpy()
    q64, k64, v64 = as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16")
    rmin, rmax = page_meta(k64, S)
    check_selection(idx, bound_scores(q64, rmin, rmax), K)
    ref = sparse_attention(q64, k64, v64, idx, S, c.scale)
    assert_close(o, ref, atol=1e-3, rel_rms=1e-4, what=f"pages P{MAX_PAGES} K{K}")
    if K == MAX_PAGES:
        assert_close(o, decode_attention(q64, k64, v64, c.scale), atol=1e-3, rel_rms=1e-4,
                     what="all 8192 pages = dense")


def longest_topk_context(D):
    """Largest n_ctx whose 10% top-k attention fits the LDS budget."""
    n = 1
    while (n + 1) + 2 * keep_count(n + 1) + 8 * D <= TOPK_LDS_FLOATS:
        n += 1
    return n


@pytest.mark.parametrize("D", [64, 128])
def test_fused_topk_at_the_lds_limit(da, D):
    import torch
    N = longest_topk_context(D)
    K = keep_count(N)
    assert N + 2 * K + 8 * D <= TOPK_LDS_FLOATS < (N + 1) + 2 * keep_count(N + 1) + 8 * D
    c = synth.dense_case([411, D, N], 1, 2, 2, D, N, "f16", "f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    o, idx = da.da_decode_attention_topk(q, k, v, K, scale=c.scale, want_idx=True)
    torch.cuda.synchronize()
    o, idx = o.cpu().numpy(), idx.cpu().numpy()
    q64, k64, v64 = as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16")
    check_selection(idx, token_scores(q64, k64), K)
    ref = sparse_attention(q64, k64, v64, idx, 1, c.scale)
    assert_close(o, ref, atol=1e-5, rel_rms=1e-4, what=f"fused topk D{D} N{N} K{K}")
    # one token more is refused before anything is launched
    c1 = synth.dense_case([411, D, N + 1], 1, 2, 2, D, N + 1, "f16", "f16")
    from sparse_kv_cache_gqa_amd._lib import DaError
    with pytest.raises(DaError, match="16384"):
        da.da_decode_attention_topk(to_dev(c1.q, "f16"), to_dev(c1.k, "f16"), to_dev(c1.v, "f16"),
                                    keep_count(N + 1), scale=c1.scale)


def test_one_kernel_page_step_at_the_lds_limit(da):
    """da_decode_attention_sparse at the edge of its LDS budget: 8192 pages of
    16 tokens and K = 217 kept pages, P + K + 2 K S + 16 D = 16377 of 16384
    floats; K = 218 is refused.  The kept set equals da_select_pages' and the
    attention matches the oracle on it."""
    import torch
    B, H, D, S, K = 1, 2, 64, 16, 217
    N = MAX_PAGES * S
    assert MAX_PAGES + K + 2 * K * S + 16 * D <= TOPK_LDS_FLOATS < MAX_PAGES + (K + 1) * (1 + 2 * S) + 16 * D
    c = synth.paged_case([211], B, H, D, N, S, K, dtype="f16")
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
    assert_close(o.cpu().numpy(), ref, atol=1e-3, rel_rms=1e-4, what=f"one-kernel pages P{MAX_PAGES} K{K}")
    with pytest.raises(da.DaError):
        da.da_decode_attention_sparse(q, kmin, kmax, k, v, S, K + 1, scale=c.scale)
