"""Seeded random shapes for decode attention over dense and uint4 caches,
each against the fp64 oracle: batch 1-3, 1-4 KV heads, G in {1, 2, 4, 8},
head_dim 64 or 128 (uint4: 128), 1-3000 tokens, every supported pair of q
and cache formats, the default split or a random multiple of 16 tokens.
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
from oracle import decode_attention, kv4_attention
from oracle.kv4 import unpack_codes
from oracle.numerics import as_f64
from gpu_util import assert_close, to_dev

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
