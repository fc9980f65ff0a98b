"""The allocation-free entry point (da_decode_attention_noalloc), through the
C ABI: its split-K partials live in the library's fixed per-GPU scratch
array.  Two calls in a row, the second on a smaller input (the array keeps
the first call's contents), each bitwise equal to da_decode_attention with a
workspace (same kernels, same split) and within the dense tolerances of the
oracle.  (The refusal of shapes beyond the array is checked on the CPU, in
tests/test_abi.py.)"""
import ctypes

import numpy as np
import pytest

import synth
from oracle import decode_attention
from oracle.numerics import as_f64
from gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu


def _noalloc_raw(da, q, k, v, out, scale):
    """Straight through the C ABI (ctypes), no binding helpers."""
    import torch
    from sparse_kv_cache_gqa_amd import _lib
    lib = _lib.load()
    B, Hq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    dt = {torch.float32: _lib.DA_F32, torch.float16: _lib.DA_F16, torch.bfloat16: _lib.DA_BF16}
    s = _lib.DaAttnShape(B, Hq, Hkv, D, N, scale, dt[q.dtype], dt[k.dtype], 0)
    st = lib.da_decode_attention_noalloc(ctypes.byref(s), ctypes.c_void_p(q.data_ptr()),
                                         ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_equals_workspace_entry_point_twice(da):
    import torch
    from sparse_kv_cache_gqa_amd import _lib
    assert _lib.load().da_decode_attention_noalloc_max_scratch() == 16 << 20
    cases = [synth.dense_case([701], 4, 32, 8, 128, 20000, "f32", "bf16"),   # 10 splits of 2048
             synth.dense_case([702], 2, 8, 2, 64, 3000, "f16", "f16")]       # smaller, 12 of 256
    for i, c in enumerate(cases):
        q, k, v = to_dev(c.q, c.q_dtype), to_dev(c.k, c.kv_dtype), to_dev(c.v, c.kv_dtype)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc_raw(da, q, k, v, out, c.scale) == _lib.DA_OK
        want = da.da_decode_attention(q, k, v, scale=c.scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.cpu().numpy().view(np.uint32)), f"call {i}"
        ref = decode_attention(as_f64(c.q, c.q_dtype), as_f64(c.k, c.kv_dtype), as_f64(c.v, c.kv_dtype),
                               c.scale)
        assert_close(got, ref, atol=1e-5, rel_rms=1e-4, what=f"noalloc call {i}")
