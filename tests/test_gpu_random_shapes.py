"""Seeded random shapes for decode attention, each against the fp64 oracle.
Dense and uint4 caches: batch 1-3, 1-4 KV heads, G in {1, 2, 4, 8},
head_dim 64 or 128 (uint4: 128), 1-3000 tokens, every supported pair of q
and cache formats, the default split or a random multiple of 16 tokens.
Page-sparse (both routes) and token top-k (one call and two): random page
sizes, kept counts, context lengths and grouped query heads, with the
selection checked by the near-tie rule and the attention on the GPU's own
set.  Chunked prefill: random chunk lengths, prefixes, head counts and
head_dim.
The cases are drawn once from a fixed seed, so every run checks the same
shapes (their parameters are in the test ids); they complement the chosen
edge cases of test_gpu_dense.py and test_gpu_kv4.py with combinations
nobody picked by hand (ragged tails at every offset, split counts that do
or do not fit one workgroup, several KV heads under grouped queries).

Bars: as in those files.  Dense: 1e-5 absolute and 1e-4 of rms.  uint4
against attention over the exact unrounded values min + code * scale (what
the kernels compute): 1e-5 absolute, and 1e-4 of rms with one query head
per KV head (fp32 weights on the VALU).  With grouped query heads each
weight enters the matrix-core products as two bf16 terms, relative error
<= 2^-18, so an output may move by up to 2^-18 times its group's value
range (~3e-5 for N(0,1) data) however small the rms of the outputs; there
the rms bar is 1e-3 (a random case measured 1.1e-4 at 4.4e-6 absolute).
Against the oracle's fp16-rounded dequantization: 1e-3 absolute and 5e-3
of rms."""
import numpy as np
import pytest

import synth
from oracle import (bound_scores, chunk_prefill_attention, decode_attention, kv4_attention, page_meta,
                    sparse_attention, token_scores)
from oracle.kv4 import unpack_codes
from oracle.numerics import as_f64
from gpu_util import assert_close, check_selection, to_dev

pytestmark = pytest.mark.gpu

_DENSE_FORMATS = [("f32", "f32"), ("f32", "f16"), ("f16", "f16"), ("f32", "bf16"), ("bf16", "bf16")]


def _draw_dense(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 3001))
        qd, kd = _DENSE_FORMATS[int(rng.integers(len(_DENSE_FORMATS)))]
        st = 0 if rng.random() < 0.5 else 16 * int(rng.integers(1, 129))
        out.append((B, G * Hkv, Hkv, D, N, qd, kd, st))
    return out


def _draw_u4(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 4, 8]))
        N = int(rng.integers(1, 3001))
        qd = "f16" if rng.random() < 0.7 else "f32"
        st = 0 if rng.random() < 0.5 else 16 * int(rng.integers(1, 129))
        out.append((B, G * Hkv, Hkv, N, qd, st))
    return out


DENSE_CASES = _draw_dense(24, 2026)
U4_CASES = _draw_u4(16, 2027)


def _ids(cases):
    return ["-".join(str(x) for x in c) for c in cases]


@pytest.mark.parametrize("B,Hq,Hkv,D,N,qd,kd,st", DENSE_CASES, ids=_ids(DENSE_CASES))
def test_random_dense(da, B, Hq, Hkv, D, N, qd, kd, st):
    import torch
    c = synth.dense_case([700, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, qd, kd)
    o = da.da_decode_attention(to_dev(c.q, qd), to_dev(c.k, kd), to_dev(c.v, kd), scale=c.scale, split_tokens=st)
    torch.cuda.synchronize()
    ref = decode_attention(as_f64(c.q, qd), as_f64(c.k, kd), as_f64(c.v, kd), c.scale)
    assert_close(o.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4,
                 what=f"dense B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} {qd}/{kd} split{st}")


def _unrounded(codes, gmin, gscale):
    c = unpack_codes(codes).astype(np.float64)
    lead, R = c.shape[:-1], c.shape[-1]
    c = c.reshape(*lead, R // 64, 64)
    x = gmin.astype(np.float64)[..., None] + c * gscale.astype(np.float64)[..., None]
    return x.reshape(*lead, R)


@pytest.mark.parametrize("B,Hq,Hkv,N,qd,st", U4_CASES, ids=_ids(U4_CASES))
def test_random_uint4(da, B, Hq, Hkv, N, qd, st):
    import torch
    c = synth.dense_case([701, B, Hq, Hkv, N], B, Hq, Hkv, 128, N, qd, "f16")
    kq = da.da_quantize_kv4(to_dev(c.k, "f16"))
    vq = da.da_quantize_kv4(to_dev(c.v, "f16"))
    o = da.da_decode_attention_kv4(to_dev(c.q, qd), *kq, *vq, scale=c.scale, split_tokens=st)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    kq = [t.cpu().numpy() for t in kq]
    vq = [t.cpu().numpy() for t in vq]
    q64 = as_f64(c.q, qd)
    what = f"uint4 B{B} Hq{Hq} Hkv{Hkv} N{N} {qd} split{st}"
    rel = 1e-4 if Hq == Hkv else 1e-3
    assert_close(o, decode_attention(q64, _unrounded(*kq), _unrounded(*vq), c.scale), atol=1e-5, rel_rms=rel,
                 what=what + " vs unrounded dequant")
    assert_close(o, kv4_attention(q64, *kq, *vq, c.scale), atol=1e-3, rel_rms=5e-3, what=what + " vs oracle")


def _draw_sparse(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        dt = "f16" if rng.random() < 0.6 else "bf16"
        S = int(rng.choice([1, 2, 4, 8, 16, 32]))
        N = int(rng.integers(1, 6001))
        P = -(-N // S)
        # the one-kernel route's LDS: P + K + 2 K S + 16 D floats <= 16384
        kmax = min(P, (16384 - P - 16 * D) // (1 + 2 * S))
        K = int(rng.integers(1, kmax + 1))
        out.append((B, G * Hkv, Hkv, D, N, S, K, dt))
    return out


SPARSE_CASES = _draw_sparse(16, 2028)


@pytest.mark.parametrize("B,Hq,Hkv,D,N,S,K,dt", SPARSE_CASES, ids=_ids(SPARSE_CASES))
def test_random_page_sparse(da, B, Hq, Hkv, D, N, S, K, dt):
    import torch
    G = Hq // Hkv
    c = synth.dense_case([702, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, dt, dt)
    q, k, v = to_dev(c.q, dt), to_dev(c.k, dt), to_dev(c.v, dt)
    kmin, kmax = da.da_build_page_meta(k, S)
    idx2 = da.da_select_pages(q, kmin, kmax, S, K, N)
    o2 = da.da_decode_attention_paged(q, k, v, idx2, S, scale=c.scale)
    o1, idx1 = da.da_decode_attention_sparse(q, kmin, kmax, k, v, S, K, scale=c.scale, want_idx=True)
    torch.cuda.synchronize()
    idx1, idx2 = idx1.cpu().numpy(), idx2.cpu().numpy()
    assert np.array_equal(idx1, idx2), "the two routes keep different pages"
    q64 = as_f64(c.q, dt)
    k64 = np.repeat(as_f64(c.k, dt), G, axis=1)
    v64 = np.repeat(as_f64(c.v, dt), G, axis=1)
    check_selection(idx1, bound_scores(q64, *page_meta(k64, S)), K)
    ref = sparse_attention(q64, k64, v64, idx1, S, c.scale)
    what = f"pages B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} S{S} K{K} {dt}"
    assert_close(o1.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=what + " one kernel")
    assert_close(o2.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=what + " two calls")


_TOKEN_FORMATS = [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16"), ("f32", "f16")]


def _draw_tokens(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 4001))
        qd, kd = _TOKEN_FORMATS[int(rng.integers(len(_TOKEN_FORMATS)))]
        K = int(rng.integers(1, N + 1))
        out.append((B, G * Hkv, Hkv, D, N, K, qd, kd))
    return out


TOKEN_CASES = _draw_tokens(12, 2029)


@pytest.mark.parametrize("B,Hq,Hkv,D,N,K,qd,kd", TOKEN_CASES, ids=_ids(TOKEN_CASES))
def test_random_token_topk(da, B, Hq, Hkv, D, N, K, qd, kd):
    import torch
    G = Hq // Hkv
    c = synth.dense_case([703, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, qd, kd)
    q, k, v = to_dev(c.q, qd), to_dev(c.k, kd), to_dev(c.v, kd)
    o1, idx1 = da.da_decode_attention_topk(q, k, v, K, scale=c.scale, want_idx=True)
    idx2 = da.da_select_tokens(q, k, K)
    o2 = da.da_decode_attention_paged(q, k, v, idx2, 1, scale=c.scale)
    torch.cuda.synchronize()
    idx1, idx2 = idx1.cpu().numpy(), idx2.cpu().numpy()
    assert np.array_equal(idx1, idx2), "the two routes keep different tokens"
    q64 = as_f64(c.q, qd)
    k64 = np.repeat(as_f64(c.k, kd), G, axis=1)
    v64 = np.repeat(as_f64(c.v, kd), G, axis=1)
    check_selection(idx1, token_scores(q64, k64), K)
    ref = sparse_attention(q64, k64, v64, idx1, 1, c.scale)
    what = f"tokens B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} K{K} {qd}/{kd}"
    assert_close(o1.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=what + " one kernel")
    assert_close(o2.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what=what + " two calls")


def _draw_prefill(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 600))
        P = int(rng.choice([0, int(rng.integers(1, 1500))]))
        dt = "bf16" if rng.random() < 0.6 else "f16"
        out.append((B, G * Hkv, Hkv, C, P, D, dt))
    return out


PREFILL_CASES = _draw_prefill(10, 2030)


@pytest.mark.parametrize("B,Hq,Hkv,C,P,D,dt", PREFILL_CASES, ids=_ids(PREFILL_CASES))
def test_random_prefill(da, B, Hq, Hkv, C, P, D, dt):
    """Bars of test_gpu_prefill.py: 1e-4 absolute and 1e-4 of rms (each
    probability enters the second product as two 16-bit terms)."""
    import torch
    c = synth.prefill_case([704, B, Hq, Hkv, C, P, D], B, Hq, Hkv, C, P, D, dt)
    o = da.da_prefill_attention(to_dev(c.q, dt), to_dev(c.k, dt), to_dev(c.v, dt), scale=c.scale)
    torch.cuda.synchronize()
    ref = chunk_prefill_attention(as_f64(c.q, dt), as_f64(c.k, dt), as_f64(c.v, dt), c.scale, P)
    assert_close(o.cpu().numpy(), ref, atol=1e-4, rel_rms=1e-4,
                 what=f"prefill B{B} Hq{Hq} Hkv{Hkv} C{C} P{P} D{D} {dt}")
