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


def assert_close(got, ref, atol, rel_rms=None, what=""):
    r = report(got, ref)
    print(f"[parity] {what} {r}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r["max_abs"] <= atol, f"{what}: max |err| {r['max_abs']:.3e} > {atol:.1e}"
    if rel_rms is not None:
        assert r["max_rel_rms"] <= rel_rms, f"{what}: max|err|/rms {r['max_rel_rms']:.3e} > {rel_rms:.1e}"
    return r
