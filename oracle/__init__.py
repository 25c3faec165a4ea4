"""Plain CPU oracle for dynamic-sparse (DSA-style) attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this
package: only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library (no kernels, headers, tables or helpers); the two
meet only at the seeded inputs drawn by the `synthetic` package.

What it computes follows the page "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理
全解析" (ruibaoantu.com), cited below as [DSA-page], section 2 "稀疏注意力DSA适配":
  §2.1  before each layer's attention, every cached key is scored against the query and a
        reduction keeps the top-K key indices;
  §2.2  the KV cache lives in fixed blocks of contiguous tokens, and the selected rows are
        gathered out of those blocks before computing;
  §2.3  prefill and decode run the same selection + gather + attention, with different
        parallel shapes;
  §2.4  vision tokens form a sequence prefix that is always attended in full and never
        enters the sparse screening; a KV dynamic allocator hands out and takes back cache
        blocks with an independent block map per layer and head.
Dense causal attention is the special case where every causal key is selected.

Everything is numpy in float64 (integers in int64). Parity status of each function is
listed in oracle/dsa.py.
"""
from .dsa import (  # noqa: F401
    bf16_to_f64,
    query_position,
    group_query_heads,
    candidate_keys,
    forced_keys,
    page_rows,
    append_rows,
    allocate_blocks,
    release_blocks,
    index_scores,
    index_scores_many,
    topk_select,
    selection_thresholds,
    INT32_MIN,
    INT32_MAX,
    index_list,
    hybrid_index_list,
    attend,
    attend_causal_many,
    dsa_query,
    dense_query,
)
