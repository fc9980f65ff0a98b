"""Chunked prefill attention (HeadInfer) on the GPU against the fp64 oracle.

Tolerance, from the arithmetic: the products q.k of bf16/fp16 values are
exact in fp32 and summed in fp32; each probability enters the second product
as two 16-bit terms (relative error <= 2^-16 for bf16), accumulated in fp32.
The output error is then ~2^-16 of the value magnitudes: |err| <= 1e-4
absolute and max|err| / rms(reference) <= 1e-4 (measured maxima are quoted
in the test output)."""
import numpy as np
import pytest

import synth
from oracle import chunk_prefill_attention, decode_attention
from oracle.numerics import as_f64
from gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu


def make(tag, B, Hq, Hkv, C, P, D, dt):
    """q for the chunk's C positions; k, v for all P + C positions."""
    c = synth.prefill_case(tag, B, Hq, Hkv, C, P, D, dt)
    return c.q, c.k, c.v


def run(da, q, k, v, dt, scale):
    import torch
    o = da.da_prefill_attention(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy()


CASES = [
    # B, Hq, Hkv, C, prefix, D, dtype
    (1, 2, 1, 100, 0, 64, "bf16"),        # one ragged workgroup, no prefix
    (1, 4, 2, 300, 200, 128, "bf16"),     # prefix, GQA, ragged last block
    (2, 2, 2, 128, 64, 64, "f16"),
    (1, 8, 8, 257, 1000, 128, "bf16"),    # MHA, longer prefix
    (1, 4, 1, 1, 500, 128, "bf16"),       # a single query: decode over 501 tokens
    (1, 2, 1, 64, 0, 128, "f16"),
    (2, 8, 4, 600, 100, 64, "bf16"),      # 8 (batch, KV head) units: one die each
]


@pytest.mark.parametrize("B,Hq,Hkv,C,P,D,dt", CASES)
def test_prefill_matches_oracle(da, B, Hq, Hkv, C, P, D, dt):
    q, k, v = make([700, B, Hq, Hkv, C, P, D], B, Hq, Hkv, C, P, D, dt)
    scale = 1.0 / np.sqrt(D)
    got = run(da, q, k, v, dt, scale)
    ref = chunk_prefill_attention(as_f64(q, dt), as_f64(k, dt), as_f64(v, dt), scale, P)
    assert_close(got, ref, atol=1e-4, rel_rms=1e-4, what=f"prefill B{B} Hq{Hq} Hkv{Hkv} C{C} P{P} D{D} {dt}")


def test_two_chunks_equal_one_bitwise(da):
    """HeadInfer's chunking: a chunk of 256 queries, and the same queries as
    two chunks of 128 (the second after the first as prefix), give the same
    bits (each query sees the same tiles in the same order)."""
    import torch
    B, Hq, Hkv, D = 1, 4, 2, 128
    q, k, v = make([701], B, Hq, Hkv, 256, 0, D, "bf16")
    whole = run(da, q, k, v, "bf16", 0.1)
    first = run(da, q[:, :, :128], k[:, :, :128], v[:, :, :128], "bf16", 0.1)
    second = run(da, q[:, :, 128:], k, v, "bf16", 0.1)
    both = np.concatenate([first, second], axis=2)
    assert np.array_equal(both.view(np.uint32), whole.view(np.uint32))


def test_llama3_8b_chunk_sampled(da):
    """A 10K-token chunk after a 10K prefix, Llama-3-8B attention heads
    (32 query / 8 KV heads, D 128, bf16), sampled queries against the decode
    oracle over their visible tokens."""
    B, Hq, Hkv, C, P, D = 1, 32, 8, 10240, 10240, 128
    q, k, v = make([702], B, Hq, Hkv, C, P, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    got = run(da, q, k, v, "bf16", scale)
    rng = np.random.default_rng(703)
    picks = [(0, 0), (31, C - 1), (5, 127), (6, 128)] + [(int(h), int(i)) for h, i in
                                                       zip(rng.integers(0, Hq, 6), rng.integers(0, C, 6))]
    for h, i in picks:
        t = P + i + 1
        kv = h // (Hq // Hkv)
        ref = decode_attention(as_f64(q[:, h:h + 1, i], "bf16"), as_f64(k[:, kv:kv + 1, :t], "bf16"),
                               as_f64(v[:, kv:kv + 1, :t], "bf16"), scale)
        assert_close(got[0, h, i], ref[0, 0], atol=1e-4, rel_rms=1e-4, what=f"llama chunk h{h} i{i}")
