"""Pins for the dense / GQA decode-attention oracle and the head-wise driver.

Each check is independent of the oracle's own formula: an independent library
implementation (torch's scaled_dot_product_attention on CPU in float64), closed
forms (one token, two tokens as a logistic blend, zero query, constant values),
structural invariants (token permutation, score shift, GQA head mapping,
batch independence) and a 50-digit brute force.  The split-K partials and
their merge are pinned the same way: merged partials against torch's
attention for ragged, single-token and whole-range splits, and the partial
of one split against its closed form.
"""
import math

import numpy as np
import pytest

import synth
from oracle import decode_attention, headwise_attention, merge_partials, split_partials
from oracle.numerics import as_f64

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rand(seed, B, Hq, Hkv, D, N):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    return q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,D,N", [(2, 8, 2, 16, 37), (1, 4, 1, 64, 256),
                                           (3, 6, 6, 8, 1), (2, 8, 1, 32, 100)])
def test_matches_torch_sdpa_float64(B, Hq, Hkv, D, N):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    q, k, v = _rand(B * 1000 + N, B, Hq, Hkv, D, N)
    G = Hq // Hkv
    tq = torch.from_numpy(q)[:, :, None, :]                       # [B,Hq,1,D]
    tk = torch.from_numpy(k).repeat_interleave(G, dim=1).contiguous()
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1).contiguous()
    ref = F.scaled_dot_product_attention(tq, tk, tv)[:, :, 0, :].numpy()
    o = decode_attention(q, k, v, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_single_token_returns_its_value():
    q, k, v = _rand(1, 2, 4, 2, 16, 1)
    o = decode_attention(q, k, v, 0.25)
    for j in range(4):
        np.testing.assert_array_equal(o[:, j], v[:, j // 2, 0])


def test_two_tokens_logistic_blend():
    # softmax over two scores is a logistic function of their difference
    rng = np.random.default_rng(7)
    D = 8
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, 2, D))
    v = rng.standard_normal((1, 1, 2, D))
    scale = 0.3
    d = scale * (float(q[0, 0] @ k[0, 0, 1]) - float(q[0, 0] @ k[0, 0, 0]))
    w1 = 1.0 / (1.0 + math.exp(-d))
    want = v[0, 0, 0] * (1.0 - w1) + v[0, 0, 1] * w1
    o = decode_attention(q, k, v, scale)
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_value():
    q, k, v = _rand(2, 2, 4, 2, 8, 50)
    q[:] = 0.0
    o = decode_attention(q, k, v, 0.5)
    for j in range(4):
        np.testing.assert_allclose(o[:, j], v[:, j // 2].mean(axis=1), atol=1e-14)


def test_constant_values_pass_through():
    q, k, v = _rand(3, 1, 2, 1, 8, 40)
    c = np.arange(8, dtype=np.float64) - 3.5
    v[:] = c
    o = decode_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[0, 0], c, atol=1e-13)
    np.testing.assert_allclose(o[0, 1], c, atol=1e-13)


def test_gqa_head_mapping_is_contiguous_groups():
    # KV head h carries the constant value (h+1); query head j must see KV
    # head j // G (not j % Hkv).
    B, Hq, Hkv, D, N = 2, 8, 4, 4, 9
    q, k, v = _rand(4, B, Hq, Hkv, D, N)
    for b in range(B):
        for h in range(Hkv):
            v[b, h] = 10 * b + h + 1
    o = decode_attention(q, k, v, 0.5)
    G = Hq // Hkv
    for b in range(B):
        for j in range(Hq):
            np.testing.assert_allclose(o[b, j], 10 * b + j // G + 1, atol=1e-12)


def test_token_permutation_invariance():
    q, k, v = _rand(5, 2, 4, 2, 16, 33)
    perm = np.random.default_rng(1).permutation(33)
    o1 = decode_attention(q, k, v, 0.25)
    o2 = decode_attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-14)


def test_score_shift_invariance():
    # moving every key by c * q / |q|^2 adds the same c * scale to every score
    q, k, v = _rand(6, 1, 1, 1, 16, 20)
    qq = q[0, 0]
    k2 = k + 3.0 * qq / (qq @ qq)
    o1 = decode_attention(q, k, v, 0.7)
    o2 = decode_attention(q, k2, v, 0.7)
    np.testing.assert_allclose(o1, o2, atol=1e-13)


def test_scale_matters_and_peaked_softmax_picks_the_argmax():
    q, k, v = _rand(7, 1, 1, 1, 16, 30)
    k[0, 0, 11] = 40.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    o = decode_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[0, 0], v[0, 0, 11], atol=1e-12)
    o_flat = decode_attention(q, k, v, 1e-9)          # near-uniform weights
    np.testing.assert_allclose(o_flat[0, 0], v[0, 0].mean(axis=0), atol=1e-7)


def test_batch_rows_are_independent():
    q, k, v = _rand(8, 3, 4, 2, 8, 17)
    o = decode_attention(q, k, v, 0.4)
    k2 = k.copy()
    v2 = v.copy()
    k2[1] += 5.0
    v2[1] *= -2.0
    o2 = decode_attention(q, k2, v2, 0.4)
    np.testing.assert_array_equal(o[0], o2[0])
    np.testing.assert_array_equal(o[2], o2[2])


def test_tiny_workload_against_50_digit_brute_force():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    c = synth.workload1()
    q, k, v = as_f64(c.q, "f32"), as_f64(c.k, "f32"), as_f64(c.v, "f32")
    o = decode_attention(q, k, v, c.scale)
    sc = mpmath.mpf(1) / mpmath.sqrt(64)
    for j in (0, 3):
        qs = [mpmath.mpf(float(x)) for x in q[0, j]]
        s = [sc * mpmath.fsum(qs[d] * mpmath.mpf(float(k[0, 0, i, d]))
                              for d in range(64)) for i in range(256)]
        w = [mpmath.exp(x) for x in s]
        Z = mpmath.fsum(w)
        for d in (0, 17, 63):
            want = mpmath.fsum(w[i] * mpmath.mpf(float(v[0, 0, i, d]))
                               for i in range(256)) / Z
            assert abs(float(want) - o[0, j, d]) <= 1e-12


def test_headwise_equals_all_heads_at_once():
    spec = synth.small_headwise(n_layers=2, n_kv_heads=2, n_q_heads=4, batch=2,
                                head_dim=16, n_ctx=45)
    q = as_f64(spec.q(), spec.q_dtype)
    ks = [[None] * 2 for _ in range(2)]
    vs = [[None] * 2 for _ in range(2)]
    for l in range(2):
        for h in range(2):
            kk, vv = spec.head(l, h)
            ks[l][h] = as_f64(kk, "bf16")
            vs[l][h] = as_f64(vv, "bf16")
    o = headwise_attention(q, ks, vs, 0.25)
    for l in range(2):
        kall = np.stack(ks[l], axis=1)       # [B][Hkv][N][D]
        vall = np.stack(vs[l], axis=1)
        ref = decode_attention(q[l], kall, vall, 0.25)
        np.testing.assert_array_equal(o[l], ref)


def _sdpa(q, k, v):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    G = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(q)[:, :, None, :]
    tk = torch.from_numpy(k).repeat_interleave(G, dim=1).contiguous()
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1).contiguous()
    return F.scaled_dot_product_attention(tq, tk, tv)[:, :, 0, :].numpy()


@pytest.mark.parametrize("S", [1, 7, 16, 37, 64])
def test_merged_split_partials_match_torch_sdpa(S):
    q, k, v = _rand(500 + S, 2, 8, 2, 16, 37)
    u, m, l = split_partials(q, k, v, 0.25, S)
    assert u.shape == (2, 8, -(-37 // S), 16)
    np.testing.assert_allclose(merge_partials(u, m, l), _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_one_split_partial_is_max_sum_and_unnormalised_output():
    q, k, v = _rand(510, 1, 4, 2, 8, 20)
    u, m, l = split_partials(q, k, v, 1.0 / math.sqrt(8), 20)
    torch = pytest.importorskip("torch")
    for j in range(4):
        h = j // 2
        x = (torch.from_numpy(k[0, h]) @ torch.from_numpy(q[0, j])).numpy() / math.sqrt(8)
        assert m[0, j, 0] == pytest.approx(x.max(), abs=1e-14)
        assert l[0, j, 0] >= 1.0
    np.testing.assert_allclose(u[..., 0, :] / l[..., 0, None], _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_single_token_splits_carry_their_score_and_value():
    q, k, v = _rand(511, 1, 2, 1, 4, 3)
    u, m, l = split_partials(q, k, v, 0.5, 1)
    for i in range(3):
        assert m[0, 0, i] == pytest.approx(0.5 * float(q[0, 0] @ k[0, 0, i]), abs=1e-14)
        assert l[0, 0, i] == 1.0
        np.testing.assert_array_equal(u[0, 0, i], v[0, 0, i])


def test_merge_ignores_split_order_and_empty_splits():
    q, k, v = _rand(512, 1, 4, 1, 8, 50)
    u, m, l = split_partials(q, k, v, 0.3, 8)
    o = merge_partials(u, m, l)
    perm = np.random.default_rng(0).permutation(u.shape[2])
    np.testing.assert_allclose(merge_partials(u[:, :, perm], m[:, :, perm], l[:, :, perm]), o,
                               rtol=0, atol=1e-14)
    ue = np.concatenate([u, np.zeros_like(u[:, :, :1])], axis=2)
    me = np.concatenate([m, np.full_like(m[:, :, :1], -np.inf)], axis=2)
    le = np.concatenate([l, np.zeros_like(l[:, :, :1])], axis=2)
    np.testing.assert_allclose(merge_partials(ue, me, le), o, rtol=0, atol=1e-15)
