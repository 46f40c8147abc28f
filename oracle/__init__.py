"""CPU oracle for the DSA indexer -> top-k -> sparse MLA attention path under IndexCache.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and shares no
code, table or helper with it.

Everything is plain NumPy in float64, evaluated row by row straight from the
definitions on the source pages.  Citations use two page titles:

  [IDX] Jerry's Blog, "注意力机制中的 Index：从位置下标到预算检索"
        (attention indices: dense attention §1, sparse attention §2, the top-k
        error decomposition §3, DeepSeek-V3.2 lightning indexer §4, GLM-5 index
        mask and deterministic top-k §6.4-§6.5, index-quality metrics §8)
  [IC]  "读懂 IndexCache：从 DSA 的选词开销到跨层索引复用"
        (F/S layer roles §1.1, the cache update loop and the {2,5,8} example §1.2,
        the multi-layer distillation loss §3.1)

Modules: formats (storage formats), dsa (indexer, top-k, attention, IndexCache loop,
index-quality metrics, the sparse-training indexer loss), upstream (the indexer's
projections, key LayerNorm, rotary encoding, cache append; [IDX] §6.4, §4), csa (the
compressed-block selection of [IDX] §5).

Every function here is pinned by tests under tests/ against closed forms,
hand-derived fixtures, brute force and library routines (see test_oracle_*.py).
"""
from .formats import decode_bf16, decode_e4m3fn, e4m3fn_table, dequant_rows, encode_e4m3fn, quantize_fp8_rows
from .dsa import (indexer_row, indexer_row_int2, topk_row, attn_row, dense_attn_row,
                  indexcache_plan, indexcache_forward, RoleError, tolerance_row,
                  captured_mass, overlap, head_mean_distribution, captured_mass_at_k, recall_at_k,
                  sparse_attention_weights, indexer_kl_row, multilayer_kl)

__all__ = ["decode_bf16", "decode_e4m3fn", "e4m3fn_table", "dequant_rows", "encode_e4m3fn", "quantize_fp8_rows", "indexer_row",
           "indexer_row_int2", "topk_row", "attn_row", "dense_attn_row", "indexcache_plan",
           "indexcache_forward", "RoleError", "tolerance_row", "captured_mass", "overlap",
           "head_mean_distribution", "captured_mass_at_k", "recall_at_k", "sparse_attention_weights",
           "indexer_kl_row", "multilayer_kl"]
