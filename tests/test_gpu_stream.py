"""Head-wise streamed decode on the GPU (HeadInfer): K/V of each (layer, KV
head) in pinned host memory, copied into two ping-pong device buffers on a copy
stream while attention runs on the compute stream.  Checked against the
oracle's head-by-head driver, and bitwise against da_decode_attention on the
same data resident in device memory."""
import numpy as np
import pytest

import synth
from oracle import headwise_attention
from oracle.numerics import as_f64
from gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu


def host_heads(spec):
    import torch
    ks, vs, k64, v64 = [], [], [], []
    for l in range(spec.n_layers):
        k64.append([])
        v64.append([])
        for h in range(spec.n_kv_heads):
            k, v = spec.head(l, h)
            tk = torch.empty(k.shape, dtype=torch.bfloat16, pin_memory=True)
            tv = torch.empty(v.shape, dtype=torch.bfloat16, pin_memory=True)
            tk.view(torch.int16).numpy()[...] = k.view(np.int16)
            tv.view(torch.int16).numpy()[...] = v.view(np.int16)
            ks.append(tk)
            vs.append(tv)
            k64[-1].append(as_f64(k, "bf16"))
            v64[-1].append(as_f64(v, "bf16"))
    return ks, vs, k64, v64


def run_stream(da, spec, hpc, ks, vs):
    import torch
    hs = da.HeadwiseStream(spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                           spec.n_ctx, da.DA_F32, da.DA_BF16, heads_per_chunk=hpc)
    buf0 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    buf1 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    q = to_dev(spec.q(), "f32")
    out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(16, hs.workspace_bytes), dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    cpy = torch.cuda.Stream()
    cpy.wait_stream(comp)
    hs.da_stream_headwise(ks, vs, buf0, buf1, q, out, ws, comp, cpy)
    torch.cuda.synchronize()
    hs.close()
    return q, out.cpu().numpy()


@pytest.mark.parametrize("hpc", [1, 2])
def test_stream_matches_oracle_and_resident_path(da, hpc):
    import torch
    spec = synth.small_headwise(n_layers=3, n_kv_heads=2, n_q_heads=8, batch=2, head_dim=64,
                                n_ctx=1000)
    ks, vs, k64, v64 = host_heads(spec)
    q, got = run_stream(da, spec, hpc, ks, vs)
    ref = headwise_attention(as_f64(spec.q(), "f32"), k64, v64, 1.0 / np.sqrt(64))
    assert_close(got, ref, atol=1e-5, rel_rms=1e-4, what=f"stream hpc{hpc}")
    H = spec.n_kv_heads
    for l in range(spec.n_layers):
        kl = torch.stack([ks[l * H + h] for h in range(H)], dim=1).cuda()   # [B][Hkv][N][D]
        vl = torch.stack([vs[l * H + h] for h in range(H)], dim=1).cuda()
        o = da.da_decode_attention(q[l].contiguous(), kl.contiguous(), vl.contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy(), got[l]), f"layer {l}: not bitwise equal"


def test_not_pinned_is_rejected(da):
    import torch
    spec = synth.small_headwise(n_layers=1, n_kv_heads=2, n_q_heads=4, batch=1, head_dim=64,
                                n_ctx=100)
    ks = [torch.zeros((1, 100, 64), dtype=torch.bfloat16) for _ in range(2)]   # pageable
    vs = [torch.zeros((1, 100, 64), dtype=torch.bfloat16) for _ in range(2)]
    with pytest.raises(da.DaError) as e:
        run_stream(da, spec, 1, ks, vs)
    assert e.value.status == da.DA_E_NOT_PINNED


def test_workload5_shape_one_layer(da):
    """HeadInfer shape at full context (N = 2^20, 8 KV heads, 32 query heads,
    bf16) for one layer: two layer-heads carry the seeded data and are checked
    against the oracle; the other six hold zeros, whose output must be 0."""
    import torch
    spec = synth.HeadwiseSpec(n_layers=1)
    ks, vs = [], []
    real = {0: None, 7: None}
    for h in range(spec.n_kv_heads):
        tk = torch.zeros((1, spec.n_ctx, 128), dtype=torch.bfloat16, pin_memory=True)
        tv = torch.zeros((1, spec.n_ctx, 128), dtype=torch.bfloat16, pin_memory=True)
        if h in real:
            spec.head(0, h, tk.view(torch.int16).numpy().view(np.uint16),
                      tv.view(torch.int16).numpy().view(np.uint16))
        ks.append(tk)
        vs.append(tv)
    q, got = run_stream(da, spec, 1, ks, vs)
    q64 = as_f64(spec.q(), "f32")
    for h in real:
        k64 = as_f64(ks[h].view(torch.int16).numpy().view(np.uint16), "bf16")
        v64 = as_f64(vs[h].view(torch.int16).numpy().view(np.uint16), "bf16")
        ref = headwise_attention(q64[:, :, 4 * h:4 * h + 4], [[k64]], [[v64]], 1.0 / np.sqrt(128))
        assert_close(got[:, :, 4 * h:4 * h + 4], ref, atol=1e-3, rel_rms=1e-4, what=f"w5 head {h}")
    for h in range(spec.n_kv_heads):
        if h not in real:
            assert not np.any(got[:, :, 4 * h:4 * h + 4]), f"zero head {h}"


def test_append_new_token_then_stream(da):
    """The per-step append: the new token's K/V rows go device-to-host into
    row `length` of every host cache, the length grows by one, and the next
    streamed step attends over the grown context (equal to the oracle and,
    bitwise, to resident attention over the same rows)."""
    import torch
    spec = synth.small_headwise(n_layers=2, n_kv_heads=2, n_q_heads=4, batch=3, head_dim=64,
                                n_ctx=300, tag=51)
    ks, vs, k64, v64 = host_heads(spec)
    L, H, B, D = spec.n_layers, spec.n_kv_heads, spec.batch, spec.head_dim
    pos = 298
    # the new token's rows, as a projection would leave them: [L][B][Hkv][D]
    k_new = torch.stack([torch.stack([ks[l * H + h][:, pos] for h in range(H)], 1) for l in range(L)])
    v_new = torch.stack([torch.stack([vs[l * H + h][:, pos] for h in range(H)], 1) for l in range(L)])
    keep_k = [t[:, pos:].clone() for t in ks]
    for t in ks + vs:
        t[:, pos:] = 0
    hs = da.HeadwiseStream(B, spec.n_q_heads, H, D, spec.n_ctx, da.DA_F32, da.DA_BF16)
    hs.set_length(pos)
    assert hs.length == pos
    cpy = torch.cuda.Stream()
    hs.append(k_new.cuda(), v_new.cuda(), ks, vs, stream=cpy)
    cpy.synchronize()
    assert hs.length == pos + 1
    for i, t in enumerate(ks):
        assert torch.equal(t[:, pos], keep_k[i][:, 0])
        assert torch.count_nonzero(t[:, pos + 1:].float()) == 0

    buf0 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    buf1 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    q = to_dev(spec.q(), "f32")
    out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(16, hs.workspace_bytes), dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    cpy.wait_stream(comp)
    hs.da_stream_headwise(ks, vs, buf0, buf1, q, out, ws, comp, cpy)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    n = pos + 1
    ref = headwise_attention(as_f64(spec.q(), "f32"), [[k[:, :n] for k in kl] for kl in k64],
                             [[v[:, :n] for v in vl] for vl in v64], 1.0 / np.sqrt(D))
    assert_close(got, ref, atol=1e-5, rel_rms=1e-4, what="stream after append")
    for l in range(L):
        kres = torch.stack([ks[l * H + h][:, :n] for h in range(H)], 1).contiguous().cuda()
        vres = torch.stack([vs[l * H + h][:, :n] for h in range(H)], 1).contiguous().cuda()
        o = da.da_decode_attention(q[l], kres, vres)
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy().view(np.uint32), got[l].view(np.uint32))

    hs.append(k_new.cuda(), v_new.cuda(), ks, vs, stream=cpy)      # row 299: full now
    cpy.synchronize()
    assert hs.length == spec.n_ctx
    with pytest.raises(da.DaError):
        hs.append(k_new.cuda(), v_new.cuda(), ks, vs, stream=cpy)
    hs.close()


def test_workspace_covers_every_attended_length(da):
    """The default split size grows in steps with the attended length, so a
    shorter length can need more splits than the capacity (cap 4097: 9 splits
    of 512; length 4096: 16 splits of 256).  The context's workspace size
    covers every length: a call at length 4096 writes nothing past it (a
    guard region after it keeps its pattern) and matches resident attention
    over the same rows bitwise."""
    import torch
    spec = synth.small_headwise(n_layers=1, n_kv_heads=1, n_q_heads=4, batch=1, head_dim=128,
                                n_ctx=4097, tag=52)
    ks, vs, k64, v64 = host_heads(spec)
    n = 4096
    hs = da.HeadwiseStream(1, 4, 1, 128, spec.n_ctx, da.DA_F32, da.DA_BF16)
    hs.set_length(n)
    need_4096 = 4 * 16 * (128 + 4) * 4            # 4 query-head rows x 16 splits of 256
    ws_bytes = hs.workspace_bytes
    assert ws_bytes >= need_4096
    guard = 1 << 16
    ws_all = torch.full((ws_bytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = ws_all[:ws_bytes]
    buf0 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    buf1 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    q = to_dev(spec.q(), "f32")
    out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    comp = torch.cuda.current_stream()
    cpy = torch.cuda.Stream()
    cpy.wait_stream(comp)
    hs.da_stream_headwise(ks, vs, buf0, buf1, q, out, ws, comp, cpy)
    torch.cuda.synchronize()
    hs.close()
    assert bool((ws_all[ws_bytes:] == 0xA5).all()), "written past the workspace"
    ref = headwise_attention(as_f64(spec.q(), "f32"), [[k64[0][0][:, :n]]], [[v64[0][0][:, :n]]],
                             1.0 / np.sqrt(128))
    assert_close(out.cpu().numpy(), ref, atol=1e-5, rel_rms=1e-4, what="stream at length 4096 of 4097")
    kl = ks[0][:, :n].unsqueeze(1).cuda().contiguous()
    vl = vs[0][:, :n].unsqueeze(1).cuda().contiguous()
    o = da.da_decode_attention(q[0].contiguous(), kl, vl)
    torch.cuda.synchronize()
    assert np.array_equal(o.cpu().numpy(), out.cpu().numpy()[0])
