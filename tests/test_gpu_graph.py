"""Library calls captured in a HIP graph: every replay, with eager work and
synchronisations between replays, equals the eager result bitwise (the graph
holds the same kernels on the same buffers; nothing the library enqueues is a
memset)."""
import numpy as np
import pytest

import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_dense_graph_replays(da):
    import torch
    c = synth.dense_case([400], 2, 8, 2, 128, 3000, "f32", "bf16")
    q, k, v = to_dev(c.q, "f32"), to_dev(c.k, "bf16"), to_dev(c.v, "bf16")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.zeros(da.da_decode_attention_workspace(2, 8, 2, 128, 3000), dtype=torch.uint8,
                     device="cuda")
    g = capture(torch, lambda: da.da_decode_attention(q, k, v, out=out, ws=ws))
    for i in range(4):
        q.mul_(0.75).add_(0.1)                      # eager work between replays
        torch.cuda.synchronize()
        want = da.da_decode_attention(q, k, v)      # eager, its own buffers
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}"


def test_paged_graph_replays(da):
    import torch
    c = synth.paged_case([401], 2, 4, 64, 2000, 16, 20, dtype="f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, 16)
    idx = torch.empty((2, 4, 20), dtype=torch.int32, device="cuda")
    out = torch.empty((2, 4, 64), dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")

    def step():
        da.da_select_pages(q, kmin, kmax, 16, 20, 2000, page_idx=idx)
        da.da_decode_attention_paged(q, k, v, idx, 16, out=out, ws=ws)

    g = capture(torch, step)
    for i in range(3):
        q.copy_(torch.flip(q, dims=[1]))            # eager work: new queries
        torch.cuda.synchronize()
        want_idx = da.da_select_pages(q, kmin, kmax, 16, 20, 2000)
        want = da.da_decode_attention_paged(q, k, v, want_idx, 16)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want_idx) and torch.equal(out, want), f"replay {i}"


def _replays_equal_eager(torch, g, out, mutate, eager, n=3):
    for i in range(n):
        mutate()                                    # eager work between replays
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}"


@pytest.mark.parametrize("G", [1, 4])
def test_kv4_graph_replays(da, G):
    """uint4 attention (one query head per KV head, and grouped heads with
    the matrix-core P.V and its LDS tiles) as captured by the benchmark."""
    import torch
    c = synth.dense_case([402, G], 2, 2 * G, 2, 128, 2500, "f16", "f16")
    q = to_dev(c.q, "f16")
    kq = da.da_quantize_kv4(to_dev(c.k, "f16"))
    vq = da.da_quantize_kv4(to_dev(c.v, "f16"))
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    g = capture(torch, lambda: da.da_decode_attention_kv4(q, *kq, *vq, out=out, ws=ws))
    _replays_equal_eager(torch, g, out, lambda: q.copy_(torch.flip(q, dims=[1])),
                         lambda: da.da_decode_attention_kv4(q, *kq, *vq))


def test_page_step_one_kernel_graph_replays(da):
    """The one-kernel page step (bound scores, top-K, attention) as captured
    by the benchmark."""
    import torch
    c = synth.paged_case([403], 2, 4, 64, 3000, 16, 30, dtype="f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    kmin, kmax = da.da_build_page_meta(k, 16)
    out = torch.empty((2, 4, 64), dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: da.da_decode_attention_sparse(q, kmin, kmax, k, v, 16, 30, out=out))
    _replays_equal_eager(torch, g, out, lambda: q.copy_(torch.flip(q, dims=[1])),
                         lambda: da.da_decode_attention_sparse(q, kmin, kmax, k, v, 16, 30))


def test_token_topk_graph_replays(da):
    """Token top-k attention in one kernel as captured by the benchmark."""
    import torch
    c = synth.dense_case([404], 2, 3, 3, 128, 1024, "f16", "f16")
    q, k, v = to_dev(c.q, "f16"), to_dev(c.k, "f16"), to_dev(c.v, "f16")
    K = da.da_token_keep_count(1024)
    out = torch.empty((2, 3, 128), dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: da.da_decode_attention_topk(q, k, v, K, out=out))
    _replays_equal_eager(torch, g, out, lambda: q.copy_(torch.flip(q, dims=[1])),
                         lambda: da.da_decode_attention_topk(q, k, v, K))


def test_prefill_graph_replays(da):
    """Chunked prefill captured in a graph (a caller that replays a layer step)."""
    import torch
    c = synth.prefill_case([405], 1, 4, 2, 300, 200, 128, "bf16")
    q, k, v = to_dev(c.q, "bf16"), to_dev(c.k, "bf16"), to_dev(c.v, "bf16")
    out = torch.empty((1, 4, 300, 128), dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: da.da_prefill_attention(q, k, v, out=out))
    _replays_equal_eager(torch, g, out, lambda: q.copy_(torch.flip(q, dims=[2])),
                         lambda: da.da_prefill_attention(q, k, v))
