"""Pins for the chunked prefill attention oracle (HeadInfer).

Independent of the oracle's own formula: torch's scaled_dot_product_attention
in float64 (causal, and with an explicit mask for a chunk after a prefix);
a one-query chunk equals decode attention over the visible tokens; and
HeadInfer's chunking claim itself -- one chunk of 2C queries gives the same
outputs as two chunks of C, the second with the first as its prefix."""
import math

import numpy as np
import pytest

from oracle import chunk_prefill_attention, decode_attention


def _rand(seed, B, Hq, Hkv, C, P, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, C, D)), rng.standard_normal((B, Hkv, P + C, D)),
            rng.standard_normal((B, Hkv, P + C, D)))


def _sdpa(q, k, v, mask):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    G = q.shape[1] // k.shape[1]
    tk = torch.from_numpy(k).repeat_interleave(G, dim=1).contiguous()
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1).contiguous()
    if mask is None:
        return F.scaled_dot_product_attention(torch.from_numpy(q), tk, tv, is_causal=True).numpy()
    return F.scaled_dot_product_attention(torch.from_numpy(q), tk, tv,
                                          attn_mask=torch.from_numpy(mask)).numpy()


@pytest.mark.parametrize("B,Hq,Hkv,C,D", [(1, 2, 1, 37, 16), (2, 8, 2, 20, 32)])
def test_no_prefix_matches_causal_sdpa(B, Hq, Hkv, C, D):
    q, k, v = _rand(600 + C, B, Hq, Hkv, C, 0, D)
    o = chunk_prefill_attention(q, k, v, 1.0 / math.sqrt(D), 0)
    np.testing.assert_allclose(o, _sdpa(q, k, v, None), rtol=0, atol=1e-12)


def test_prefix_matches_masked_sdpa():
    B, Hq, Hkv, C, P, D = 2, 4, 2, 13, 29, 16
    q, k, v = _rand(601, B, Hq, Hkv, C, P, D)
    o = chunk_prefill_attention(q, k, v, 1.0 / math.sqrt(D), P)
    mask = np.arange(P + C)[None, :] <= (P + np.arange(C))[:, None]
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask), rtol=0, atol=1e-12)


def test_each_query_is_decode_over_its_visible_tokens():
    B, Hq, Hkv, C, P, D = 1, 4, 1, 6, 10, 8
    q, k, v = _rand(602, B, Hq, Hkv, C, P, D)
    o = chunk_prefill_attention(q, k, v, 0.3, P)
    for i in range(C):
        t = P + i + 1
        ref = decode_attention(q[:, :, i], k[:, :, :t], v[:, :, :t], 0.3)
        np.testing.assert_allclose(o[:, :, i], ref, rtol=0, atol=1e-13)


def test_first_query_without_prefix_returns_first_value():
    q, k, v = _rand(603, 1, 2, 2, 5, 0, 8)
    o = chunk_prefill_attention(q, k, v, 0.5, 0)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])


def test_two_chunks_equal_one():
    B, Hq, Hkv, C, D = 1, 4, 2, 12, 16
    q, k, v = _rand(604, B, Hq, Hkv, 2 * C, 0, D)
    whole = chunk_prefill_attention(q, k, v, 0.25, 0)
    first = chunk_prefill_attention(q[:, :, :C], k[:, :, :C], v[:, :, :C], 0.25, 0)
    second = chunk_prefill_attention(q[:, :, C:], k, v, 0.25, C)
    np.testing.assert_allclose(np.concatenate([first, second], axis=2), whole, rtol=0, atol=1e-13)
