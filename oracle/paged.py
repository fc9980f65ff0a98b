"""Query-aware page selection and sparse attention (TinyServe), fp64.

Follows TinyServe (papercache.org digest), section "方法细节":

* the cache is cut into P = ceil(t / S) pages of S tokens;
* each page keeps per-channel minimum m_j and maximum M_j of its keys;
* the relevance of page j to query q is sum_i (q_i M_{j,i} if q_i >= 0 else
  q_i m_{j,i}), an upper bound on max_{k in page} q . k;
* the K pages with the largest relevance are kept (S_t = TopK, |S_t| = K);
* attention runs over the tokens of the kept pages only, softmax normalised
  over them (Algorithm 1, steps 3 and 4).

Readings where the page is silent: a partial last page holds only its valid
tokens (metadata and attention ignore positions >= N); ties in the relevance go
to the lower page index; the kept pages are listed in ascending order; the
softmax uses the same 1/sqrt(D) scale as dense attention (ranking is unchanged
by a positive scale, so selection uses the unscaled score).
"""
from __future__ import annotations

import numpy as np


def page_meta(k: np.ndarray, page_size: int):
    """Per-page, per-channel min and max of the keys.

    k [B][H][N][D] (any float type; min/max is exact).  Returns kmin, kmax
    [B][H][P][D] with P = ceil(N / S); page j covers tokens [jS, min((j+1)S, N)).
    """
    B, H, N, D = k.shape
    S = page_size
    P = -(-N // S)
    kmin = np.empty((B, H, P, D), dtype=k.dtype)
    kmax = np.empty((B, H, P, D), dtype=k.dtype)
    for j in range(P):
        blk = k[:, :, j * S:min((j + 1) * S, N), :]
        kmin[:, :, j, :] = blk.min(axis=2)
        kmax[:, :, j, :] = blk.max(axis=2)
    return kmin, kmax


def bound_scores(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """r[b,h,j] = sum_d (q_d * kmax_d if q_d >= 0 else q_d * kmin_d).

    q [B][H][D], kmin/kmax [B][H][P][D], float64.  Returns [B][H][P].
    """
    pos = q >= 0
    sel = np.where(pos[:, :, None, :], kmax, kmin)     # per channel: M or m
    return np.einsum("bhd,bhpd->bhp", q, sel)


def topk_pages(r: np.ndarray, top_k: int) -> np.ndarray:
    """Indices of the top_k largest scores per (b, h), ascending.

    Order is by (-score, page index), so equal scores keep the lower index.
    Returns int32 [B][H][top_k].
    """
    B, H, P = r.shape
    if not 1 <= top_k <= P:
        raise ValueError("top_k must be in [1, P]")
    out = np.empty((B, H, top_k), dtype=np.int32)
    idx = np.arange(P)
    for b in range(B):
        for h in range(H):
            order = np.lexsort((idx, -r[b, h]))    # primary key: -score
            out[b, h] = np.sort(order[:top_k])
    return out


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     page_idx: np.ndarray, page_size: int,
                     scale: float) -> np.ndarray:
    """Attention of q[b,h] over the tokens of the listed pages only.

    q [B][H][D], k/v [B][H][N][D] float64 (one KV head per query head),
    page_idx [B][H][K].  Tokens at or beyond N (partial last page) are skipped,
    and so is a listed page index outside [0, ceil(N/S)): such a page holds no
    token of the cache.  A list with no page inside the cache has nothing to
    attend, and its output is zero.
    """
    B, H, D = q.shape
    N = k.shape[2]
    S = page_size
    P = -(-N // S)
    o = np.empty((B, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            toks = [t for j in page_idx[b, h] if 0 <= int(j) < P
                    for t in range(int(j) * S, min((int(j) + 1) * S, N))]
            if not toks:
                o[b, h] = 0.0
                continue
            kk = k[b, h, toks]
            vv = v[b, h, toks]
            s = scale * (kk @ q[b, h])
            e = np.exp(s - s.max())
            o[b, h] = (e @ vv) / e.sum()
    return o
