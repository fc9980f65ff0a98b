"""Pins for the page-metadata, bound-score, top-K and sparse-attention oracle.

Independent checks: explicit loops on tiny arrays (metadata), the maximum of a
linear form over a box is attained at a corner (bound score, by enumerating
all 2^D corners), the bound dominates every true q.k of its page and is exact
for one-token pages, Python's sorted() on (-score, index) (top-K), and the
reductions of sparse attention to dense attention (all pages; one-token pages).
"""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import (bound_scores, decode_attention, page_meta, sparse_attention,
                    topk_pages)
from oracle.numerics import as_f64
from oracle.sizes import tinyserve_memory_fraction


def test_page_meta_matches_loops_with_partial_last_page():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, 3, 23, 5)).astype(np.float16)
    S = 4
    kmin, kmax = page_meta(k, S)
    assert kmin.shape == (2, 3, 6, 5)
    for b in range(2):
        for h in range(3):
            for j in range(6):
                for d in range(5):
                    vals = [float(k[b, h, t, d]) for t in range(j * S, min(j * S + S, 23))]
                    assert float(kmin[b, h, j, d]) == min(vals)
                    assert float(kmax[b, h, j, d]) == max(vals)


def test_bound_is_max_over_box_corners():
    rng = np.random.default_rng(1)
    D = 6
    q = rng.standard_normal((1, 1, D))
    lo = rng.standard_normal((1, 1, 3, D))
    hi = lo + rng.random((1, 1, 3, D)) * 2
    r = bound_scores(q, lo, hi)
    for j in range(3):
        best = max(sum(q[0, 0, d] * (hi if c[d] else lo)[0, 0, j, d] for d in range(D))
                   for c in itertools.product((0, 1), repeat=D))
        assert abs(r[0, 0, j] - best) < 1e-12


def test_bound_dominates_every_key_of_its_page():
    c = synth.paged_case(99, 2, 3, 16, 200, 8, 4)
    q = as_f64(c.q, "f16")
    k = as_f64(c.k, "f16")
    kmin, kmax = page_meta(k, 8)
    r = bound_scores(q, kmin, kmax)
    qk = np.einsum("bhd,bhnd->bhn", q, k)
    P = r.shape[-1]
    for j in range(P):
        page_max = qk[:, :, j * 8:min(j * 8 + 8, 200)].max(axis=-1)
        slack = np.abs(q).sum(-1) * np.abs(k).max() * 1e-12
        assert np.all(r[:, :, j] >= page_max - slack)


def test_one_token_pages_bound_equals_dot_product():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 2, 8))
    k = rng.standard_normal((2, 2, 11, 8))
    kmin, kmax = page_meta(k, 1)
    r = bound_scores(q, kmin, kmax)
    np.testing.assert_allclose(r, np.einsum("bhd,bhnd->bhn", q, k), atol=1e-13)


def test_topk_matches_sorted_with_ties():
    rng = np.random.default_rng(3)
    r = rng.integers(0, 6, size=(2, 3, 17)).astype(np.float64)   # many ties
    out = topk_pages(r, 5)
    for b in range(2):
        for h in range(3):
            order = sorted(range(17), key=lambda j: (-r[b, h, j], j))
            assert list(out[b, h]) == sorted(order[:5])


def test_topk_all_pages_and_bad_k():
    r = np.random.default_rng(4).standard_normal((1, 2, 9))
    assert np.array_equal(topk_pages(r, 9)[0, 0], np.arange(9))
    with pytest.raises(ValueError):
        topk_pages(r, 10)
    with pytest.raises(ValueError):
        topk_pages(r, 0)


def test_sparse_with_all_pages_equals_dense():
    c = synth.paged_case(98, 2, 3, 16, 70, 16, 5)
    q, k, v = as_f64(c.q, "f16"), as_f64(c.k, "f16"), as_f64(c.v, "f16")
    P = 5
    idx = np.broadcast_to(np.arange(P, dtype=np.int32), (2, 3, P))
    o = sparse_attention(q, k, v, idx, 16, c.scale)
    ref = decode_attention(q, k, v, c.scale)
    np.testing.assert_allclose(o, ref, atol=1e-14)


def test_one_token_pages_all_selected_equals_dense():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 2, 13, 8))
    v = rng.standard_normal((1, 2, 13, 8))
    kmin, kmax = page_meta(k, 1)
    idx = topk_pages(bound_scores(q, kmin, kmax), 13)
    o = sparse_attention(q, k, v, idx, 1, 0.3)
    np.testing.assert_allclose(o, decode_attention(q, k, v, 0.3), atol=1e-14)


def test_sparse_single_page_is_attention_over_that_page():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 4))
    k = rng.standard_normal((1, 1, 10, 4))
    v = rng.standard_normal((1, 1, 10, 4))
    idx = np.array([[[2]]], dtype=np.int32)             # tokens 8, 9 (partial page)
    o = sparse_attention(q, k, v, idx, 4, 1.0)
    s = [float(q[0, 0] @ k[0, 0, t]) for t in (8, 9)]
    w = [math.exp(x - max(s)) for x in s]
    want = (w[0] * v[0, 0, 8] + w[1] * v[0, 0, 9]) / (w[0] + w[1])
    np.testing.assert_allclose(o[0, 0], want, atol=1e-14)


def test_sparse_out_of_range_pages_hold_no_tokens():
    """Listed page indices outside [0, P) name no token of the cache: with them
    the result is attention over the in-range pages, computed by hand; a list
    of out-of-range pages only attends nothing and gives zero."""
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 2, 4))
    k = rng.standard_normal((1, 2, 10, 4))
    v = rng.standard_normal((1, 2, 10, 4))
    idx = np.array([[[-1, 1, 3, 40], [-7, 3, 4, 1 << 30]]], dtype=np.int32)   # P = 3 (page 4)
    o = sparse_attention(q, k, v, idx, 4, 1.0)
    # head 0: page 1 = tokens 4..7; pages -1, 3 and 40 are outside the cache
    s = [float(q[0, 0] @ k[0, 0, t]) for t in range(4, 8)]
    w = [math.exp(x - max(s)) for x in s]
    want = sum(wi * v[0, 0, t] for wi, t in zip(w, range(4, 8))) / sum(w)
    np.testing.assert_allclose(o[0, 0], want, atol=1e-14)
    assert np.all(o[0, 1] == 0.0)


def test_planted_page_is_selected():
    c = synth.paged_case(97, 1, 2, 16, 256, 16, 3, boost_frac=0.0)
    q = as_f64(c.q, "f16")
    k = as_f64(c.k, "f16")
    u = q[0, 1] / np.linalg.norm(q[0, 1])
    k[0, 1, 5 * 16:6 * 16] = 30.0 * u                  # page 5 of head 1
    kmin, kmax = page_meta(k, 16)
    idx = topk_pages(bound_scores(q, kmin, kmax), 3)
    assert 5 in idx[0, 1]


def test_tinyserve_memory_fraction_is_one_eighth_at_workload3():
    # page 16, 128 pages of a 32768-token cache, no reuse
    assert tinyserve_memory_fraction(16, 128, 32768, 1.0) == 0.125
