"""Dense / GQA decode attention on the GPU against the fp64 oracle.

Tolerances: the required bar is |err| <= 1e-3 absolute on the fp32 output;
on top of it these tests hold max|err| / rms(reference) <= 1e-4 (outputs of
N(0,1) data are small, rms ~ sqrt(e/N)), and small shapes hold 1e-5 absolute.
"""
import numpy as np
import pytest

import synth
from oracle import decode_attention
from oracle.numerics import as_f64
from gpu_util import assert_close, each_row, to_dev

pytestmark = pytest.mark.gpu


def run(da, c: synth.DenseCase, split_tokens=0):
    import torch
    q = to_dev(c.q, c.q_dtype)
    k = to_dev(c.k, c.kv_dtype)
    v = to_dev(c.v, c.kv_dtype)
    o = da.da_decode_attention(q, k, v, scale=c.scale, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def oracle_of(c: synth.DenseCase):
    return decode_attention(as_f64(c.q, c.q_dtype), as_f64(c.k, c.kv_dtype),
                            as_f64(c.v, c.kv_dtype), c.scale)


def test_workload1_tiny_fp32(da):
    c = synth.workload1()
    assert_close(run(da, c), oracle_of(c), atol=1e-5, rel_rms=1e-4, what="tiny fp32")


CASES = [
    # B, Hq, Hkv, D, N, q, kv, split_tokens
    (2, 8, 2, 128, 1000, "f32", "bf16", 0),     # ragged tail, 2 splits
    (1, 4, 1, 64, 1, "f32", "f32", 0),          # a single token
    (3, 16, 2, 64, 777, "f16", "f16", 128),     # G = 8, fp16 q
    (2, 4, 4, 128, 300, "f32", "f16", 16),      # MHA, 19 splits of 16
    (2, 8, 8, 64, 2049, "bf16", "bf16", 0),     # bf16 q, one token past a split
    (1, 8, 1, 128, 5000, "f32", "bf16", 1024),  # G = 8 with fp32 q split in two terms
    (2, 2, 1, 64, 129, "f32", "f32", 32),
    (1, 32, 8, 128, 4096, "f32", "bf16", 512),  # the Llama-3-8B layer, short context
    (2, 16, 8, 128, 333, "f32", "f32", 0),      # fp32 cache, G = 2
    (1, 8, 2, 64, 70, "f32", "f16", 64),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,N,qd,kd,st", CASES)
def test_small_shapes(da, B, Hq, Hkv, D, N, qd, kd, st):
    c = synth.dense_case([100, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, qd, kd)
    assert_close(run(da, c, st), oracle_of(c), atol=1e-5, rel_rms=1e-4,
                 what=f"B{B} Hq{Hq} Hkv{Hkv} D{D} N{N} {qd}/{kd} split{st}")


def test_peaked_softmax_and_large_scores(da):
    # one token per head scores ~ +60 above the rest: every other weight
    # underflows; exercise the -inf / rescale paths
    c = synth.dense_case([101], 2, 8, 2, 128, 900, "f32", "f32")
    q64 = as_f64(c.q, "f32")
    for b in range(2):
        for h in range(2):
            u = q64[b, h * 4] / np.linalg.norm(q64[b, h * 4])
            c.k[b, h, 613] = (60.0 * u).astype(np.float32)     # score ~ +60 for head h*4
    assert_close(run(da, c, 64), oracle_of(c), atol=1e-5, rel_rms=1e-4, what="peaked")


def test_constant_values_and_zero_query(da):
    c = synth.dense_case([102], 1, 4, 2, 64, 500, "f32", "bf16")
    c.q[0, 0] = 0.0
    c.v[0, 1] = c.v[0, 1, 7]                     # KV head 1: every value row equal
    got = run(da, c)
    ref = oracle_of(c)
    assert_close(got, ref, atol=1e-5, rel_rms=1e-4, what="const")
    np.testing.assert_allclose(got[0, 2], as_f64(c.v[0, 1, 7], "bf16"), atol=1e-6)


def test_deterministic(da):
    c = synth.dense_case([103], 2, 8, 2, 128, 3000, "f32", "bf16")
    a = run(da, c)
    b = run(da, c)
    assert np.array_equal(a, b)


def test_split_sizes_agree(da):
    c = synth.dense_case([104], 1, 8, 2, 128, 2500, "f32", "bf16")
    ref = oracle_of(c)
    for st in (16, 48, 512, 4096):
        assert_close(run(da, c, st), ref, atol=1e-5, rel_rms=1e-4, what=f"split {st}")


def test_workload2_full_size_every_row(da):
    """The Llama-3-8B layer at 32K context, in the benchmark's launch
    configuration (default split): every (batch row, query head) against the
    oracle, computed one batch row at a time."""
    c = synth.workload2()
    got = run(da, c)
    B = c.q.shape[0]

    def row(b):
        ref = decode_attention(as_f64(c.q[b:b + 1], "f32"), as_f64(c.k[b:b + 1], "bf16"),
                               as_f64(c.v[b:b + 1], "bf16"), c.scale)
        return assert_close(got[b:b + 1], ref, atol=1e-3, rel_rms=1e-4, what=f"w2 row {b}")

    rs = each_row(row, B)
    print(f"[parity] w2 all {B}x32 rows: max |err| {max(r['max_abs'] for r in rs):.2e}", flush=True)


def _upload(c):
    q = to_dev(c.q, c.q_dtype)
    k = to_dev(c.k, c.kv_dtype)
    v = to_dev(c.v, c.kv_dtype)
    return q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,D,N,qd,kd,st", [
    (2, 8, 2, 128, 1000, "f32", "bf16", 256),   # 4 splits, ragged last
    (1, 4, 4, 64, 300, "f16", "f16", 64),       # MHA fp16, 5 splits
    (1, 16, 2, 64, 77, "f32", "f32", 32),       # fp32 cache, G = 8
])
def test_partials_match_oracle(da, B, Hq, Hkv, D, N, qd, kd, st):
    """The split-K pass on its own: every split's (u, m, l) against the
    oracle's partials (the kernel keeps m in base 2)."""
    import torch
    from oracle import split_partials
    c = synth.dense_case([105, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, qd, kd)
    q, k, v = _upload(c)
    ws = da.da_decode_attention_partials(q, k, v, scale=c.scale, split_tokens=st)
    torch.cuda.synchronize()
    ws = ws.cpu().numpy().astype(np.float64)
    u, m, l = split_partials(as_f64(c.q, qd), as_f64(c.k, kd), as_f64(c.v, kd), c.scale, st)
    assert ws.shape == (B, Hq, u.shape[2], D + 4)
    m_got = ws[..., D] * np.log(2.0)
    np.testing.assert_allclose(m_got, m, rtol=0, atol=2e-6 * max(1.0, np.abs(m).max()))
    np.testing.assert_allclose(ws[..., D + 1], l, rtol=2e-6, atol=0)
    assert_close(ws[..., :D], u, atol=2e-6 * np.abs(u).max(), what=f"partials u split {st}")


@pytest.mark.parametrize("ns,D", [(1, 64), (3, 128), (16, 128), (7, 64), (20, 64), (32, 128), (33, 64), (100, 128)])
def test_merge_matches_oracle(da, ns, D):
    """The cross-split merge on its own, on seeded partials with empty splits
    (m = -inf) and a wide spread of maxima."""
    import torch
    from oracle import merge_partials
    rng = np.random.default_rng([106, ns, D])
    rows = 37
    m2 = rng.uniform(-20.0, 20.0, (rows, ns))
    l = rng.uniform(1.0, 50.0, (rows, ns))
    u = rng.standard_normal((rows, ns, D)) * l[..., None]
    if ns > 1:
        empty = rng.random((rows, ns)) < 0.2
        empty[:, 0] = False
        m2[empty] = -np.inf
        l[empty] = 0.0
        u[empty] = 0.0
    part = np.zeros((rows, ns, D + 4), dtype=np.float32)
    part[..., :D] = u
    part[..., D] = m2
    part[..., D + 1] = l
    got = da.da_merge_partials(torch.from_numpy(part).cuda())
    torch.cuda.synchronize()
    p64 = part.astype(np.float64)
    ref = merge_partials(p64[..., :D], p64[..., D] * np.log(2.0), p64[..., D + 1])
    assert_close(got.cpu().numpy(), ref, atol=2e-6 * np.abs(ref).max(), what=f"merge ns{ns} D{D}")


@pytest.mark.parametrize("ns,D", [(4, 128), (32, 128), (32, 64)])
def test_merge_kernels_agree_bitwise(da, ns, D):
    """The merge kernels for up to 4, up to 32 and more splits do the same
    arithmetic in the same order: merging ns splits, and the same splits
    followed by one empty split (m = -inf, l = 0, u = 0; it crosses into the
    next kernel), must give the same bits."""
    import torch
    rng = np.random.default_rng([108, ns, D])
    rows = 29
    part = np.zeros((rows, ns + 1, D + 4), dtype=np.float32)
    part[:, :ns, :D] = rng.standard_normal((rows, ns, D))
    part[:, :ns, D] = rng.uniform(-20.0, 20.0, (rows, ns))
    part[:, :ns, D + 1] = rng.uniform(1.0, 50.0, (rows, ns))
    part[:, ns, D] = -np.inf
    a = da.da_merge_partials(torch.from_numpy(np.ascontiguousarray(part[:, :ns])).cuda())
    b = da.da_merge_partials(torch.from_numpy(part).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("B,Hq,Hkv,D,N,qd,kd", [
    (64, 8, 4, 64, 1000, "f32", "bf16"),    # 256 units x 4 splits: one 4-wave workgroup each
    (128, 4, 2, 128, 600, "f32", "bf16"),   # 3 splits
    (1, 4, 1, 64, 200, "f32", "f32"),       # a single split
    (32, 16, 8, 128, 700, "f16", "f16"),    # 3 splits, G = 2
])
def test_in_workgroup_merge_equals_merge_kernel_bitwise(da, B, Hq, Hkv, D, N, qd, kd):
    """When a (b, h) has at most four splits they run as the waves of one
    workgroup and merge in LDS; the result must carry the same bits as the
    partial pass followed by the merge kernel, and match the oracle."""
    import torch
    c = synth.dense_case([107, B, Hq, Hkv, D, N], B, Hq, Hkv, D, N, qd, kd)
    q, k, v = _upload(c)
    assert da.da_decode_attention_n_split(B, Hq, Hkv, D, N) <= 4
    fused = da.da_decode_attention(q, k, v, scale=c.scale)
    two = da.da_merge_partials(da.da_decode_attention_partials(q, k, v, scale=c.scale))
    torch.cuda.synchronize()
    a = fused.cpu().numpy()
    b = two.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert_close(a, oracle_of(c), atol=1e-5, rel_rms=1e-4, what=f"fused B{B} N{N}")
