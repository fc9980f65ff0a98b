"""Helpers for the GPU parity tests: upload storage arrays, error metrics."""
from __future__ import annotations

import numpy as np


def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def report(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got.astype(np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return {"max_abs": float(err.max()), "rms_ref": rms,
            "max_rel_rms": float(err.max() / rms) if rms > 0 else float(err.max())}


def assert_close(got, ref, atol, rel_rms=None, what="", quiet=False):
    r = report(got, ref)
    if not quiet:
        print(f"[parity] {what} {r}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r["max_abs"] <= atol, f"{what}: max |err| {r['max_abs']:.3e} > {atol:.1e}"
    if rel_rms is not None:
        assert r["max_rel_rms"] <= rel_rms, f"{what}: max|err|/rms {r['max_rel_rms']:.3e} > {rel_rms:.1e}"
    return r


def from_dev(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_selection(got_idx: np.ndarray, r: np.ndarray, top_k: int, rel_band: float = 1e-5):
    """GPU-selected page sets against oracle scores r [B][H][P] (fp64).

    The sets must be ascending, unique, in range, of size top_k, and equal to
    the oracle's top-k set except for pages whose oracle score lies within
    rel_band * |s_K| of the oracle's k-th score s_K (near-ties that fp32
    accumulation may order differently)."""
    B, H, P = r.shape
    n_diff = 0
    for b in range(B):
        for h in range(H):
            g = got_idx[b, h].astype(np.int64)
            assert np.all(np.diff(g) > 0), f"({b},{h}) not strictly ascending"
            assert g.min() >= 0 and g.max() < P
            order = np.lexsort((np.arange(P), -r[b, h]))
            ref = set(order[:top_k].tolist())
            sK = r[b, h, order[top_k - 1]]
            band = rel_band * abs(sK) + 1e-12
            for j in ref.symmetric_difference(g.tolist()):
                assert abs(r[b, h, j] - sK) <= band, \
                    f"({b},{h}) page {j}: score {r[b, h, j]!r} vs k-th {sK!r}"
                n_diff += 1
    return n_diff


def each_row(fn, n: int):
    """fn(0) .. fn(n-1) on a thread pool (the oracle's NumPy work releases the
    GIL), in order; for full-size checks computed one batch row at a time."""
    import concurrent.futures as cf
    import os
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    with cf.ThreadPoolExecutor(max(1, min(16, cores))) as ex:
        return list(ex.map(fn, range(n)))
