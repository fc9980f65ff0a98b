"""Pins for the token-level top-k sparse attention oracle (FlexGen).

Independent of the oracle's own formulas: keeping every token is dense
attention (itself pinned against torch); keeping one token returns the value
of the argmax key; the selection agrees with numpy's argsort on distinct
scores and with a planted set of large scores; ties keep the lower index;
the kept count is ceil(10% of N)."""
import math

import numpy as np
import pytest

from oracle import decode_attention, keep_count, token_scores, topk_token_attention, topk_tokens


def _rand(seed, B, H, D, N):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, D)), rng.standard_normal((B, H, N, D)),
            rng.standard_normal((B, H, N, D)))


def test_keep_count_is_ceil_of_ten_percent():
    assert keep_count(1024) == 103
    assert keep_count(1000) == 100
    assert keep_count(5) == 1
    assert keep_count(1) == 1
    assert keep_count(20, 1.0) == 20


def test_keep_all_equals_dense():
    q, k, v = _rand(1, 2, 3, 16, 40)
    o, idx = topk_token_attention(q, k, v, 40, 0.25)
    np.testing.assert_array_equal(idx[0, 0], np.arange(40))
    np.testing.assert_allclose(o, decode_attention(q, k, v, 0.25), rtol=0, atol=1e-13)


def test_keep_one_returns_value_of_best_key():
    q, k, v = _rand(2, 1, 2, 8, 30)
    o, idx = topk_token_attention(q, k, v, 1, 0.3)
    for h in range(2):
        best = int(np.argmax(k[0, h] @ q[0, h]))
        assert idx[0, h, 0] == best
        np.testing.assert_array_equal(o[0, h], v[0, h, best])


def test_selection_matches_argsort_and_is_ascending():
    q, k, _ = _rand(3, 2, 2, 8, 64)
    s = token_scores(q, k)
    np.testing.assert_allclose(s[1, 0], k[1, 0] @ q[1, 0], rtol=0, atol=1e-13)
    idx = topk_tokens(s, 7)
    for b in range(2):
        for h in range(2):
            want = np.sort(np.argsort(-s[b, h], kind="stable")[:7])
            np.testing.assert_array_equal(idx[b, h], want)


def test_planted_tokens_are_kept_and_ties_keep_lower_index():
    q, k, v = _rand(4, 1, 1, 8, 50)
    u = q[0, 0] / np.linalg.norm(q[0, 0])
    for i in (3, 17, 41):
        k[0, 0, i] = 20 * u
    _, idx = topk_token_attention(q, k, v, 3, 0.1)
    np.testing.assert_array_equal(idx[0, 0], [3, 17, 41])
    _, idx2 = topk_token_attention(q, k, v, 2, 0.1)
    np.testing.assert_array_equal(idx2[0, 0], [3, 17])


def test_bad_top_k():
    with pytest.raises(ValueError):
        topk_tokens(np.zeros((1, 1, 5)), 6)
    with pytest.raises(ValueError):
        topk_tokens(np.zeros((1, 1, 5)), 0)
