"""Chunked prefill attention (HeadInfer), fp64.

Follows HeadInfer (blog.gzher.com), section "chunked prefill 与 adaptive head
grouping": the input sequence is processed in fixed-size chunks (10K tokens
by default), each chunk building its part of the KV cache; a chunk's queries
attend to every earlier token (the cache built so far) and causally to the
chunk itself, so chunking changes the memory footprint, not the result.
The per-head equation is the one of section "核心 idea" with the causal mask
of prefill.

Readings where the page is silent (each is a choice of this library):

* query i of a chunk that starts at position `prefix` sits at position
  prefix + i and attends to positions 0 .. prefix + i (inclusive);
* grouped queries: query head j reads KV head floor(j / G), as in decode;
* the scale is 1/sqrt(D).
"""
from __future__ import annotations

import numpy as np


def chunk_prefill_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                            prefix: int) -> np.ndarray:
    """q [B][Hq][C][D] at positions prefix .. prefix + C - 1; k, v
    [B][Hkv][prefix + C][D] (the cache including the chunk).  Returns
    o [B][Hq][C][D] float64."""
    B, Hq, C, D = q.shape
    Bk, Hkv, T, Dk = k.shape
    assert (Bk, Dk) == (B, D) and v.shape == k.shape and T == prefix + C
    assert Hq % Hkv == 0
    G = Hq // Hkv
    pos = prefix + np.arange(C)
    visible = np.arange(T)[None, :] <= pos[:, None]          # [C][T]
    o = np.empty((B, Hq, C, D))
    for b in range(B):
        for j in range(Hq):
            h = j // G
            s = scale * (q[b, j] @ k[b, h].T)                  # [C][T]
            s = np.where(visible, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            o[b, j] = (e @ v[b, h]) / e.sum(axis=1, keepdims=True)
    return o
