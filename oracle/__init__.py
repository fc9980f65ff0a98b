"""CPU oracle for decode attention over a large KV cache -- TEST INFRASTRUCTURE.

A plain, slow, obviously correct fp64 NumPy statement of what the GPU library
computes.  It shares no code with the HIP path (no kernels, headers, helpers,
tables or pre/post-processing) and imports nothing from it; the only common
module is ``synth`` (seeded input draws).  Only the tests, the smoke check and
the CPU-baseline leg of the benchmark may import it; the library itself never
does.

Sources (the pages these functions follow):

* HeadInfer (blog.gzher.com, "论文阅读：HeadInfer"): per-head decode attention
  equation in section "核心 idea"; head independence, ping-pong buffers and the
  on-GPU size formula in sections "核心 idea", "三个维度的切分" and "方法：
  ping-pong memory 与异步重叠"; chunked prefill in "chunked prefill 与 adaptive
  head grouping".
* TinyServe (papercache.org, "TinyServe: Query-Aware Cache Selection"):
  standard decode equation, page partition, TopK, SparseAttn and the
  directional bounding-box score in section "方法细节" and Algorithm 1.
* FlexGen (kwkr.cn digest, section "方法细节"): 4-bit min/max quantization in
  groups of 64 along the hidden dimension, dequantized to FP16 before compute;
  sparse attention over the top 10% of the K cache per query.

Modules:

* :mod:`oracle.attention` -- dense / GQA decode attention, its split-K
  partials and their merge, head-wise driver.
* :mod:`oracle.paged` -- page metadata, bound score, top-K, sparse attention.
* :mod:`oracle.kv4` -- uint4 group quantization, dequantization, attention.
* :mod:`oracle.tokens` -- token-level top-k sparse attention (FlexGen).
* :mod:`oracle.prefill` -- chunked prefill attention (HeadInfer).

Pinning status: every function is pinned by tests against closed forms,
invariants, brute force on tiny inputs or an independent library routine (see
``tests/test_oracle_*.py``); none is "parity unpinned".
"""
from .numerics import as_f64, f64_to_f16_bits  # noqa: F401
from .attention import (decode_attention, headwise_attention,  # noqa: F401
                        split_partials, merge_partials)
from .paged import (page_meta, bound_scores, topk_pages,  # noqa: F401
                    sparse_attention)
from .kv4 import quantize_kv4, dequantize_kv4, kv4_attention  # noqa: F401
from .tokens import (keep_count, token_scores, topk_tokens,  # noqa: F401
                     topk_token_attention)
from .prefill import chunk_prefill_attention  # noqa: F401
