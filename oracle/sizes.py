"""Closed-form cache sizes and data-movement fractions printed on the pages.

* HeadInfer, section "三个维度的切分": the on-GPU cache of one head is
  2 * B * S * D_h * sizeof(dtype) (the 2 is key plus value), and the resident
  fraction of head-wise offload is alpha = 1 / (L * H).
* TinyServe, section "方法细节" (memory-efficiency model): per decode step the
  fraction of full-cache traffic moved is 1/S + rho * K * S / L.
* FlexGen, section "为什么单卡跑大模型这么难": the whole KV cache of a model is
  2 (key, value) * layers * hidden * tokens * batch * sizeof(dtype).
"""
from __future__ import annotations


def headinfer_head_bytes(batch: int, seq: int, head_dim: int, esize: int) -> int:
    return 2 * batch * seq * head_dim * esize


def headinfer_alpha(n_layers: int, n_kv_heads: int) -> float:
    return 1.0 / (n_layers * n_kv_heads)


def kv_cache_bytes(n_layers: int, hidden_kv: int, seq: int, batch: int,
                   esize: int) -> int:
    return 2 * n_layers * hidden_kv * seq * batch * esize


def tinyserve_memory_fraction(page_size: int, top_k: int, ctx: int,
                              rho: float = 1.0) -> float:
    return 1.0 / page_size + rho * top_k * page_size / ctx
