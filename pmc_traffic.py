"""Turn two rocprofv3 PMC result databases (FETCH_SIZE pass, WRITE_SIZE pass)
into calibrated HBM bytes per launch, keyed by kernel, for bench.py.

    python pmc_traffic.py FETCH_DB WRITE_DB OUT_JSON

(FETCH_DB / WRITE_DB: rocprofv3 result databases, or the
pmc_counter_collection.csv files of --output-format csv runs.)

Both runs must include the 512 MiB device-to-device copies that
`bench.py --copy-calibration` performs first (`__amd_rocclr_copyBuffer`):
each counter is scaled by (true bytes of that copy) / (what the counter read
for it).  The output records the SHA-256 of the kernel sources, so stale
figures can be recognised.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sqlite3
import statistics
import sys

PKG = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_kv_cache_gqa_amd")
COPY_KIB = 512 * 1024          # one calibration copy reads and writes 512 MiB
KERNELS = {                    # short name -> substring of the mangled kernel name
    "attn_split_llama3_8b_32k": "attn_split_kernel<2, 0, 128, 4, false, 0>",
    "select_tinyserve_32k": "select_kernel<1, 1, 64, 0>",
    "page_attention_tinyserve_32k": "select_kernel<1, 1, 64, 3>",
    "attn_split_paged_tinyserve_32k": "attn_split_kernel<1, 1, 64, 1, true, 0>",
    "attn_split_uint4_flexgen": "attn_split_kernel<3, 1, 128, 1, false, 1>",
    "topk_attention_flexgen": "select_kernel<1, 1, 128, 2>",
    "select_tokens_flexgen": "select_kernel<1, 1, 128, 1>",
    "attn_reduce": "attn_reduce_kernel",
    "attn_reduce_mid": "attn_reduce_mid_kernel",
    "attn_reduce_small": "attn_reduce_small_kernel",
}


def source_hash() -> str:
    h = hashlib.sha256()
    # the sources of the kernels in KERNELS (and what they include)
    for rel in ("csrc/kernels/attn.hip", "csrc/kernels/attn_split.h", "csrc/kernels/attn_u4.hip",
                "csrc/kernels/page.hip", "csrc/kernels/kv4.hip", "csrc/kernels/common.h", "csrc/internal.h"):
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _per_kernel(db: str, counter: str) -> dict:
    """Counter values per kernel name, from a rocprofv3 result database or
    from its CSV output (pmc_counter_collection.csv, one row per dispatch)."""
    if db.endswith(".csv"):
        with open(db, newline="") as fh:
            rows = [(r["Kernel_Name"], r["Counter_Value"]) for r in csv.DictReader(fh)
                    if r["Counter_Name"] == counter]
    else:
        con = sqlite3.connect(db)
        rows = con.execute("select name, counter_value from pmc_events where counter_name = ?",
                           (counter,)).fetchall()
    out: dict = {}
    for name, v in rows:
        out.setdefault(name, []).append(float(v))
    return out


def build(fetch_db: str, write_db: str) -> dict:
    f = _per_kernel(fetch_db, "FETCH_SIZE")
    w = _per_kernel(write_db, "WRITE_SIZE")
    cf = COPY_KIB / statistics.median(f["__amd_rocclr_copyBuffer"])
    cw = COPY_KIB / statistics.median(w["__amd_rocclr_copyBuffer"])
    res = {"source_sha256": source_hash(), "calibration": {"fetch_scale": cf, "write_scale": cw,
           "copy": "3 x 512 MiB device-to-device copies in the same process"}, "kernels": {}}
    for short, pat in KERNELS.items():
        names = [n for n in f if pat in n]
        if not names:
            continue
        n = names[0]
        res["kernels"][short] = {
            "kernel": n, "launches": len(f[n]),
            "fetch_bytes": statistics.median(f[n]) * cf * 1024,
            "write_bytes": statistics.median(w.get(n, [0.0])) * cw * 1024,
        }
    return res


if __name__ == "__main__":
    if len(sys.argv) != 4:
        print(__doc__)
        sys.exit(2)
    data = build(sys.argv[1], sys.argv[2])
    with open(sys.argv[3], "w") as fh:
        json.dump(data, fh, indent=1)
    print(json.dumps(data, indent=1))
