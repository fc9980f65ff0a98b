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


@pytest.mark.parametrize("hpc,Hkv,Hq,L", [(1, 2, 8, 3), (2, 2, 8, 3), (4, 8, 16, 2), (8, 8, 32, 2),
                                           (2, 8, 8, 1)])
def test_stream_matches_oracle_and_resident_path(da, hpc, Hkv, Hq, L):
    """Head grouping (HeadInfer's adaptive head grouping): 1, 2, 4 or 8 KV
    heads per transfer (8 of 8 = layer-wise), against the oracle and bitwise
    against resident attention over the same rows."""
    import torch
    spec = synth.small_headwise(n_layers=L, n_kv_heads=Hkv, n_q_heads=Hq, batch=2, head_dim=64,
                                n_ctx=1000, tag=50 + hpc * 10 + Hkv)
    ks, vs, k64, v64 = host_heads(spec)
    q, got = run_stream(da, spec, hpc, ks, vs)
    ref = headwise_attention(as_f64(spec.q(), "f32"), k64, v64, 1.0 / np.sqrt(64))
    assert_close(got, ref, atol=1e-5, rel_rms=1e-4, what=f"stream hpc{hpc} Hkv{Hkv} Hq{Hq}")
    H = spec.n_kv_heads
    for l in range(spec.n_layers):
        kl = torch.stack([ks[l * H + h] for h in range(H)], dim=1).cuda()   # [B][Hkv][N][D]
        vl = torch.stack([vs[l * H + h] for h in range(H)], dim=1).cuda()
        o = da.da_decode_attention(q[l].contiguous(), kl.contiguous(), vl.contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy(), got[l]), f"layer {l}: not bitwise equal"


def test_back_to_back_calls_need_no_caller_ordering(da):
    """Two steps on one context straight after each other, with different
    caches and queries, no synchronisation and no stream wait by the caller:
    the second step's first copies go into the buffers the first step's last
    attentions read, so they must wait for them.  Both outputs against the
    oracle, and bitwise against a step run on its own."""
    import torch
    specs = [synth.small_headwise(n_layers=2, n_kv_heads=2, n_q_heads=8, batch=2, head_dim=128,
                                  n_ctx=4000, tag=t) for t in (61, 62)]
    data = [host_heads(sp) for sp in specs]
    sp = specs[0]
    hs = da.HeadwiseStream(sp.batch, sp.n_q_heads, sp.n_kv_heads, sp.head_dim, sp.n_ctx, da.DA_F32,
                           da.DA_BF16)
    buf0 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    buf1 = torch.empty(hs.buffer_bytes, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(max(16, hs.workspace_bytes), dtype=torch.uint8, device="cuda")
    qs = [to_dev(x.q(), "f32") for x in specs]
    outs = [torch.zeros(q.shape, dtype=torch.float32, device="cuda") for q in qs]
    comp = torch.cuda.current_stream()
    cpy = torch.cuda.Stream()
    torch.cuda.synchronize()
    for i in range(2):
        hs.da_stream_headwise(data[i][0], data[i][1], buf0, buf1, qs[i], outs[i], ws, comp, cpy)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    for i in range(2):
        ref = headwise_attention(as_f64(specs[i].q(), "f32"), data[i][2], data[i][3], 1.0 / np.sqrt(128))
        assert_close(got[i], ref, atol=1e-5, rel_rms=1e-4, what=f"back-to-back step {i}")
    # each step alone, synchronised
    for i in range(2):
        alone = torch.zeros_like(outs[i])
        hs.da_stream_headwise(data[i][0], data[i][1], buf0, buf1, qs[i], alone, ws, comp, cpy)
        torch.cuda.synchronize()
        assert np.array_equal(alone.cpu().numpy().view(np.uint32), got[i].view(np.uint32)), f"step {i}"
    hs.close()


def test_not_pinned_is_rejected(da):
    import torch
    spec = synth.small_headwise(n_layers=1, n_kv_heads=2, n_q_heads=4, batch=1, head_dim=64,
                                n_ctx=100)
    ks = [torch.zeros((1, 100, 64), dtype=torch.bfloat16) for _ in range(2)]   # pageable
    vs = [torch.zeros((1, 100, 64), dtype=torch.bfloat16) for _ in range(2)]
    with pytest.raises(da.DaError) as e:
        run_stream(da, spec, 1, ks, vs)
    assert e.value.status == da.DA_E_NOT_PINNED


@pytest.mark.timeout(600)
def test_workload5_full_shape(da):
    """HeadInfer shape at full size, as bench.py runs it: 32 layers x 8 KV
    heads of 2^20 bf16 tokens (512 MiB per layer-head), 32 query heads, one
    step streamed through the two 512 MiB buffers.  Like the benchmark, a
    pinned pool of 16 seeded layer-heads (8 GiB) backs the 256 layer-heads of
    the step cyclically (layer-head i reads pool entry i mod 16); every entry
    holds its own seeded data.  Checked against the oracle: all 8 heads of
    layers 0 and 31 and four seeded layer-heads in between (20 of 256)."""
    import concurrent.futures as cf
    import torch
    spec = synth.HeadwiseSpec()
    L, H, POOL = spec.n_layers, spec.n_kv_heads, 16
    shp = (spec.batch, spec.n_ctx, spec.head_dim)
    pool_k = [torch.empty(shp, dtype=torch.bfloat16, pin_memory=True) for _ in range(POOL)]
    pool_v = [torch.empty(shp, dtype=torch.bfloat16, pin_memory=True) for _ in range(POOL)]

    def bits(t):
        return t.view(torch.int16).numpy().view(np.uint16)

    def fill(i):
        l, h = divmod(i, H)
        spec.head(l, h, bits(pool_k[i]), bits(pool_v[i]))

    with cf.ThreadPoolExecutor(16) as ex:
        list(ex.map(fill, range(POOL)))
    print("[w5] pool filled", flush=True)
    ks = [pool_k[i % POOL] for i in range(L * H)]
    vs = [pool_v[i % POOL] for i in range(L * H)]
    q, got = run_stream(da, spec, 1, ks, vs)
    print("[w5] step streamed", flush=True)
    rng = np.random.default_rng([42, 5, 9])
    picks = [(0, h) for h in range(H)] + [(L - 1, h) for h in range(H)]
    picks += [(int(l), int(h)) for l, h in zip(rng.choice(np.arange(1, L - 1), 4, replace=False),
                                                 rng.integers(0, H, 4))]
    q64 = as_f64(spec.q(), "f32")
    G = spec.n_q_heads // H

    def check(lh):
        l, h = lh
        p = (l * H + h) % POOL
        k64, v64 = as_f64(bits(pool_k[p]), "bf16"), as_f64(bits(pool_v[p]), "bf16")
        assert np.any(k64) and np.any(v64)
        ref = headwise_attention(q64[l:l + 1, :, G * h:G * (h + 1)], [[k64]], [[v64]],
                                 1.0 / np.sqrt(spec.head_dim))
        return assert_close(got[l:l + 1, :, G * h:G * (h + 1)], ref, atol=1e-3, rel_rms=1e-4,
                            what=f"w5 layer {l} head {h} (pool {p})")

    with cf.ThreadPoolExecutor(4) as ex:
        rs = list(ex.map(check, picks))
    print(f"[parity] w5 {len(picks)} layer-heads: max |err| {max(r['max_abs'] for r in rs):.2e}", flush=True)


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
