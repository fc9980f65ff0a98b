"""Dense / grouped-query decode attention, and the head-wise driver (fp64).

Follows the per-head decode equation of HeadInfer (section "核心 idea":
A_t^(h) = Softmax(Q_t^(h) K^(h)T / sqrt(d_k)) V^(h)) and TinyServe's standard
decode step (section "方法细节", Attn(q_t, K, V)).

Readings where the pages are silent:

* scale: 1/sqrt(D) as in HeadInfer's equation (TinyServe's omits it);
* grouped queries: query head j reads KV head floor(j / G), G = Hq / Hkv
  (HeadInfer names 8 KV heads for Llama-3-8B but not the mapping);
* every one of the N cached tokens is attended, with no mask (the current
  token's key/value is already in the cache).
"""
from __future__ import annotations

import numpy as np


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     scale: float) -> np.ndarray:
    """o[b, j] = sum_i softmax_i(scale * q[b,j] . k[b,h,i]) v[b,h,i], h = j // G.

    q [B][Hq][D], k and v [B][Hkv][N][D], all float64.  Returns [B][Hq][D].
    """
    B, Hq, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    assert (Bk, Dk) == (B, D) and v.shape == k.shape and N >= 1
    assert Hq % Hkv == 0
    G = Hq // Hkv
    o = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for j in range(Hq):
            h = j // G
            s = scale * (k[b, h] @ q[b, j])          # [N]
            m = s.max()
            e = np.exp(s - m)
            o[b, j] = (e @ v[b, h]) / e.sum()
    return o


def split_partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   split_tokens: int):
    """Flash-decode partials of each token split (the split-K form of the
    per-head equation: the softmax over all N tokens factors into per-split
    maxima, sums and unnormalised outputs).

    Split s covers tokens [s * S, min((s + 1) * S, N)), S = split_tokens.
    For every (b, query head j, split s), with h = j // G and
    x_i = scale * q[b,j] . k[b,h,i] over the split's tokens:
    m = max x_i, l = sum exp(x_i - m), u = sum exp(x_i - m) v[b,h,i].
    Returns u [B][Hq][n_split][D], m and l [B][Hq][n_split] (natural base).
    """
    B, Hq, D = q.shape
    _, Hkv, N, _ = k.shape
    G = Hq // Hkv
    S = int(split_tokens)
    ns = -(-N // S)
    u = np.zeros((B, Hq, ns, D))
    m = np.empty((B, Hq, ns))
    l = np.empty((B, Hq, ns))
    for b in range(B):
        for j in range(Hq):
            h = j // G
            for s in range(ns):
                t0, t1 = s * S, min((s + 1) * S, N)
                x = scale * (k[b, h, t0:t1] @ q[b, j])
                m[b, j, s] = x.max()
                e = np.exp(x - m[b, j, s])
                l[b, j, s] = e.sum()
                u[b, j, s] = e @ v[b, h, t0:t1]
    return u, m, l


def merge_partials(u: np.ndarray, m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Combine split partials: M = max_s m_s, L = sum_s l_s exp(m_s - M),
    o = sum_s u_s exp(m_s - M) / L.  A split with m = -inf (no tokens)
    carries no weight.  u [..., n_split, D], m and l [..., n_split]."""
    M = m.max(axis=-1, keepdims=True)
    w = np.where(np.isneginf(m), 0.0, np.exp(m - M))
    L = (w * l).sum(axis=-1)
    return (w[..., None] * u).sum(axis=-2) / L[..., None]


def headwise_attention(q: np.ndarray, k_heads, v_heads, scale: float) -> np.ndarray:
    """Head-by-head decode over a multi-layer cache (HeadInfer).

    q [L][B][Hq][D]; k_heads[l][h] and v_heads[l][h] are [B][N][D] arrays (or
    callables returning them) for layer l, KV head h.  Each (layer, KV head) is
    computed on its own, as the head-wise offload does; the result is
    concatenated into o [L][B][Hq][D].
    """
    L, B, Hq, D = q.shape
    Hkv = len(k_heads[0])
    G = Hq // Hkv
    o = np.empty((L, B, Hq, D), dtype=np.float64)
    for l in range(L):
        for h in range(Hkv):
            kh = k_heads[l][h]() if callable(k_heads[l][h]) else k_heads[l][h]
            vh = v_heads[l][h]() if callable(v_heads[l][h]) else v_heads[l][h]
            qs = q[l][:, h * G:(h + 1) * G, :]
            o[l][:, h * G:(h + 1) * G, :] = decode_attention(
                qs, kh[:, None], vh[:, None], scale)
    return o
