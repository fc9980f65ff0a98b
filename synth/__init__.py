"""Seeded synthetic inputs for decode attention over a large KV cache.

This module is the only code shared by the CPU oracle and the HIP path: it
draws random numbers and rounds them to the storage type, and nothing else.
It holds none of the method's arithmetic (no scores, softmax, page bounds,
selection or quantization).

Storage conventions (what both sides receive):

* ``f32``  -> ``numpy.float32``
* ``f16``  -> ``numpy.float16`` (IEEE binary16, rounded to nearest even)
* ``bf16`` -> ``numpy.uint16`` holding bfloat16 bit patterns (round to nearest
  even from float32)

Every array is drawn from ``numpy.random.default_rng`` with a seed list that
starts with 42 (the seed TinyServe fixes in its reproducibility notes) and the
workload number, so any slice (one batch row, one layer-head) can be drawn on
its own without drawing the rest.

Workloads (numbered as in the measurement plan):

1. tiny dense: B1, 4 query heads on 1 KV head, D64, N256, fp32 q/K/V.
2. Llama-3-8B-shaped layer: B8, 32 query / 8 KV heads, D128, N32768,
   bf16 K/V, fp32 q.
3. page-sparse (TinyServe): B32, H16 MHA, D64, N32768, fp16 K/V/q, pages of 16
   tokens; keys clustered per page, 4% of pages boosted x3.
4. uint4 KV (FlexGen): B64, H56 MHA, D128, N1024, fp16 K/V/q.
5. head-wise streamed (HeadInfer): 32 layers x 8 KV heads, B1, N 2^20, D128,
   bf16 K/V per layer-head, fp32 q [32][1][32][128].
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

SEED = 42


# ----------------------------------------------------------------------------
# storage rounding (input preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _normal(seed, shape, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _parallel_rows(fn, n: int):
    if n == 1:
        return [fn(0)]
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, range(n)))


# ----------------------------------------------------------------------------
# dense decode inputs
# ----------------------------------------------------------------------------
@dataclass
class DenseCase:
    """q [B][Hq][D]; k, v [B][Hkv][N][D] in storage form."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_dtype: str
    kv_dtype: str
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Hq, D = self.q.shape
        _, Hkv, N, _ = self.k.shape
        return B, Hq, Hkv, D, N


def dense_case(tag, B, Hq, Hkv, D, N, q_dtype="f32", kv_dtype="bf16",
               rows=None) -> DenseCase:
    """i.i.d. N(0,1) q, K, V.

    Seeds: q <- [42, *tag, 0]; K[b] <- [42, *tag, 1, b]; V[b] <- [42, *tag, 2, b].
    ``rows`` limits K/V to the listed batch rows (the others are not drawn and
    the returned arrays hold only those rows, in the order given).
    """
    tag = list(tag) if isinstance(tag, (list, tuple)) else [tag]
    q = _normal([SEED, *tag, 0], (B, Hq, D), q_dtype)
    rows = list(range(B)) if rows is None else list(rows)

    def draw(which):
        def one(i):
            return _normal([SEED, *tag, which, rows[i]], (Hkv, N, D), kv_dtype)
        return np.stack(_parallel_rows(one, len(rows)))

    k = draw(1)
    v = draw(2)
    return DenseCase(q=q, k=k, v=v, q_dtype=q_dtype, kv_dtype=kv_dtype,
                     scale=1.0 / np.sqrt(D), meta={"tag": tag, "rows": rows})


def workload1() -> DenseCase:
    """Tiny dense: B1, Hq4/Hkv1, D64, N256, fp32 everything."""
    return dense_case(1, 1, 4, 1, 64, 256, "f32", "f32")


def workload2(rows=None) -> DenseCase:
    """Llama-3-8B layer: B8, Hq32/Hkv8, D128, N32768, bf16 K/V, fp32 q."""
    return dense_case(2, 8, 32, 8, 128, 32768, "f32", "bf16", rows=rows)


# ----------------------------------------------------------------------------
# page-sparse inputs (clustered keys)
# ----------------------------------------------------------------------------
@dataclass
class PagedCase:
    q: np.ndarray      # [B][H][D] f16
    k: np.ndarray      # [B][H][N][D] f16
    v: np.ndarray      # [B][H][N][D] f16
    page_size: int
    top_k: int
    scale: float
    q_dtype: str = "f16"
    kv_dtype: str = "f16"
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, H, D = self.q.shape
        return B, H, H, D, self.k.shape[2]


def paged_case(tag, B, H, D, N, page_size, top_k, boost_frac=0.04,
               boost=3.0, noise=0.3, dtype="f16", rows=None) -> PagedCase:
    """Keys clustered by page: key = centre(page) + noise * eps.

    Per batch row b, one generator [42, *tag, 1, b] draws, in this order:
    centres [H][P][D] ~ N(0,1); then for each head h in order one permutation
    of the P pages, whose first round(boost_frac * P) entries get their centre
    multiplied by ``boost``; then eps [H][N][D] ~ N(0,1).  The key is formed in
    float32 (centre + noise * eps) and rounded once to the storage type.  A
    partial last page (N % page_size != 0) uses the centre of its page.
    V[b] <- [42, *tag, 2, b] i.i.d. N(0,1); q <- [42, *tag, 0] N(0,1).
    """
    tag = list(tag) if isinstance(tag, (list, tuple)) else [tag]
    P = -(-N // page_size)
    n_boost = int(round(boost_frac * P))
    q = _normal([SEED, *tag, 0], (B, H, D), dtype)
    rows = list(range(B)) if rows is None else list(rows)

    def keys(i):
        rng = np.random.default_rng([SEED, *tag, 1, rows[i]])
        c = rng.standard_normal((H, P, D), dtype=np.float32)
        for h in range(H):
            perm = rng.permutation(P)
            c[h, perm[:n_boost]] *= np.float32(boost)
        eps = rng.standard_normal((H, N, D), dtype=np.float32)
        page_of = np.arange(N) // page_size
        key = c[:, page_of, :] + np.float32(noise) * eps
        return to_storage(key, dtype)

    def vals(i):
        return _normal([SEED, *tag, 2, rows[i]], (H, N, D), dtype)

    k = np.stack(_parallel_rows(keys, len(rows)))
    v = np.stack(_parallel_rows(vals, len(rows)))
    return PagedCase(q=q, k=k, v=v, page_size=page_size, top_k=top_k,
                     scale=1.0 / np.sqrt(D), q_dtype=dtype, kv_dtype=dtype,
                     meta={"tag": tag, "rows": rows, "n_boost": n_boost})


def workload3(rows=None) -> PagedCase:
    """TinyServe-style: B32, H16, D64, N32768, fp16, page 16, top-128 pages."""
    return paged_case(3, 32, 16, 64, 32768, 16, 128, rows=rows)


# ----------------------------------------------------------------------------
# uint4 inputs
# ----------------------------------------------------------------------------
def workload4(rows=None) -> DenseCase:
    """FlexGen-style: B64, H56 MHA, D128, N1024, fp16 q/K/V (quantized later)."""
    return dense_case(4, 64, 56, 56, 128, 1024, "f16", "f16", rows=rows)


# ----------------------------------------------------------------------------
# chunked prefill inputs
# ----------------------------------------------------------------------------
@dataclass
class PrefillCase:
    q: np.ndarray          # [B][Hq][C][D], positions prefix .. prefix + C - 1
    k: np.ndarray          # [B][Hkv][prefix + C][D]
    v: np.ndarray
    dtype: str
    prefix: int
    scale: float


def prefill_case(tag, B, Hq, Hkv, C, prefix, D, dtype="bf16") -> PrefillCase:
    """i.i.d. N(0,1) q, K, V.  q <- [42, *tag, 0]; K <- [42, *tag, 1];
    V <- [42, *tag, 2]."""
    tag = list(tag) if isinstance(tag, (list, tuple)) else [tag]
    q = _normal([SEED, *tag, 0], (B, Hq, C, D), dtype)
    k = _normal([SEED, *tag, 1], (B, Hkv, prefix + C, D), dtype)
    v = _normal([SEED, *tag, 2], (B, Hkv, prefix + C, D), dtype)
    return PrefillCase(q=q, k=k, v=v, dtype=dtype, prefix=prefix, scale=1.0 / np.sqrt(D))


def workload6() -> PrefillCase:
    """HeadInfer chunked prefill on Llama-3-8B attention: the fourth 10K-token
    chunk (prefix 30720), 32 query / 8 KV heads, D 128, bf16."""
    return prefill_case(6, 1, 32, 8, 10240, 30720, 128, "bf16")


# ----------------------------------------------------------------------------
# head-wise streamed inputs
# ----------------------------------------------------------------------------
@dataclass
class HeadwiseSpec:
    n_layers: int = 32
    n_kv_heads: int = 8
    n_q_heads: int = 32
    batch: int = 1
    head_dim: int = 128
    n_ctx: int = 1 << 20
    kv_dtype: str = "bf16"
    q_dtype: str = "f32"
    tag: int = 5

    @property
    def head_bytes(self) -> int:
        esz = 4 if self.kv_dtype == "f32" else 2
        return self.batch * self.n_ctx * self.head_dim * esz

    def q(self) -> np.ndarray:
        """q [L][B][Hq][D] <- [42, tag, 0]."""
        return _normal([SEED, self.tag, 0],
                       (self.n_layers, self.batch, self.n_q_heads, self.head_dim),
                       self.q_dtype)

    def head(self, layer: int, kv_head: int, out_k=None, out_v=None):
        """K, V of one layer-head, [B][N][D] each.

        K <- [42, tag, 1, layer, kv_head]; V <- [42, tag, 2, layer, kv_head].
        The batch rows are drawn in one call, so (B, N, D) is the draw shape.
        """
        shp = (self.batch, self.n_ctx, self.head_dim)
        k = _normal([SEED, self.tag, 1, layer, kv_head], shp, self.kv_dtype)
        v = _normal([SEED, self.tag, 2, layer, kv_head], shp, self.kv_dtype)
        if out_k is not None:
            out_k[...] = k
            out_v[...] = v
            return out_k, out_v
        return k, v


def workload5() -> HeadwiseSpec:
    return HeadwiseSpec()


def small_headwise(n_layers=2, n_kv_heads=2, n_q_heads=8, batch=2,
                   head_dim=64, n_ctx=1000, kv_dtype="bf16", q_dtype="f32",
                   tag=50) -> HeadwiseSpec:
    return HeadwiseSpec(n_layers, n_kv_heads, n_q_heads, batch, head_dim,
                        n_ctx, kv_dtype, q_dtype, tag)
