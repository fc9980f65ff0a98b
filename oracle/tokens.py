"""Token-level top-k sparse attention (FlexGen), fp64.

Follows the FlexGen digest (kwkr.cn), section "方法细节": for each query only
the indices of the top 10% of the K cache are kept, and only the matching
subset of the V cache is loaded.

Readings where the page is silent (each is a choice of this library):

* "top 10% of the K cache" ranks tokens by the exact attention score
  q . k_i (a positive scale does not change the ranking);
* the number kept is ceil(keep * N) with keep = 0.1, at least one token;
* ties go to the lower token index and the kept indices are listed in
  ascending order (as for page selection);
* attention over the kept tokens is the softmax restricted to them and
  renormalised (the same rule as TinyServe's SparseAttn), with the dense
  scale 1/sqrt(D).
"""
from __future__ import annotations

import math

import numpy as np


def keep_count(n_ctx: int, keep: float = 0.1) -> int:
    """Tokens kept per query: ceil(keep * N), at least 1, at most N."""
    return min(n_ctx, max(1, math.ceil(keep * n_ctx - 1e-9)))


def token_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """s[b, h, i] = q[b, h] . k[b, h, i]; q [B][H][D], k [B][H][N][D]."""
    return np.einsum("bhd,bhnd->bhn", q, k)


def topk_tokens(s: np.ndarray, top_k: int) -> np.ndarray:
    """Indices of the top_k largest scores per (b, h), ascending; ties keep
    the lower index.  Returns int32 [B][H][top_k]."""
    B, H, N = s.shape
    if not 1 <= top_k <= N:
        raise ValueError("top_k must be in [1, N]")
    out = np.empty((B, H, top_k), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            ranked = sorted(range(N), key=lambda i: (-s[b, h, i], i))
            out[b, h] = sorted(ranked[:top_k])
    return out


def topk_token_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, top_k: int,
                         scale: float):
    """Attention of each query over its top_k tokens only.

    q [B][H][D], k and v [B][H][N][D] float64 (one KV head per query head).
    Returns (o [B][H][D], idx [B][H][top_k])."""
    idx = topk_tokens(token_scores(q, k), top_k)
    B, H, D = q.shape
    o = np.empty((B, H, D))
    for b in range(B):
        for h in range(H):
            kk = k[b, h, idx[b, h]]
            vv = v[b, h, idx[b, h]]
            x = scale * (kk @ q[b, h])
            e = np.exp(x - x.max())
            o[b, h] = (e @ vv) / e.sum()
    return o, idx
