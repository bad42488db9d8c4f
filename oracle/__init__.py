"""CPU oracle for the DeepSeek-V4 DSA indexer hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy (float64) versions of the operations on
the path: the weighted-ReLU MQA logits (dense bf16/fp8 keys, or keys in a
paged mxfp4/fp8 cache), the per-query top-k selection, the mxfp4 paged KV
gather, the producers of the quantized inputs (per-row fp8 quantizer,
mxfp4 cache writer) and the sparse attention that consumes the selection.  It shares no code, header, table or constant with
the HIP library; it has its own bf16 / OCP-e4m3 / E2M1 / E8M0 decoders.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never calls it.

Pins (what checks the oracle against something other than itself) live in
``tests/test_oracle_pins*.py``; every function below is pinned there.
"""
from .formats import (bf16_bits_to_f64, e4m3_to_f64, e2m1_to_f64, e8m0_to_f64,
                      f64_to_bf16_bits)
from .indexer import (indexer_logits, indexer_topk, topk_row, mxfp4_paged_gather,
                      paged_keys, indexer_logits_paged)
from .quant import (e4m3_encode, e2m1_encode, quant_fp8_rows, mxfp4_encode_rows,
                    mxfp4_cache_write)
from .attention import sparse_attention

__all__ = [
    "bf16_bits_to_f64", "e4m3_to_f64", "e2m1_to_f64", "e8m0_to_f64", "f64_to_bf16_bits",
    "indexer_logits", "indexer_topk", "topk_row", "mxfp4_paged_gather",
    "paged_keys", "indexer_logits_paged",
    "e4m3_encode", "e2m1_encode", "quant_fp8_rows", "mxfp4_encode_rows", "mxfp4_cache_write",
    "sparse_attention",
]
