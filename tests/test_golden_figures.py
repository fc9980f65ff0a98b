"""The closed-form size helpers reproduce the figures printed on the pages."""
import json
import os

from oracle.sizes import (headinfer_alpha, headinfer_head_bytes, kv_cache_bytes,
                          tinyserve_memory_fraction)

HERE = os.path.dirname(os.path.abspath(__file__))
GiB = 1 << 30


def _figs():
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        return {d["name"]: d for d in json.load(f)["figures"]}


def test_headinfer_sizes():
    f = _figs()
    a = f["headinfer_total_kv_llama3_8b_1m_bf16"]["inputs"]
    total = kv_cache_bytes(a["n_layers"], a["n_kv_heads"] * a["head_dim"], a["seq"],
                           a["batch"], a["esize"])
    assert total == f["headinfer_total_kv_llama3_8b_1m_bf16"]["value_gib"] * GiB
    b = f["headinfer_on_gpu_kv_headwise"]["inputs"]
    one = headinfer_head_bytes(b["batch"], b["seq"], b["head_dim"], b["esize"])
    assert b["buffers"] * one == f["headinfer_on_gpu_kv_headwise"]["value_gib"] * GiB
    c = f["headinfer_on_gpu_kv_layerwise"]["inputs"]
    layer = c["n_kv_heads"] * headinfer_head_bytes(c["batch"], c["seq"], c["head_dim"], c["esize"])
    assert c["buffers"] * layer == f["headinfer_on_gpu_kv_layerwise"]["value_gib"] * GiB
    assert headinfer_alpha(32, 8) == f["headinfer_alpha_headwise"]["value"]
    assert headinfer_alpha(32, 1) == f["headinfer_alpha_layerwise"]["value"]


def test_tinyserve_fraction():
    f = _figs()["tinyserve_fraction_workload3"]
    i = f["inputs"]
    assert tinyserve_memory_fraction(i["page_size"], i["top_k"], i["ctx"], i["rho"]) == f["value"]


def test_flexgen_kv_peak():
    f = _figs()["flexgen_kv_peak_opt175b"]
    i = f["inputs"]
    tib = kv_cache_bytes(i["n_layers"], i["hidden"], i["seq"], i["batch"], i["esize"]) / (1 << 40)
    assert abs(tib - f["value_tib_approx"]) < 0.05
