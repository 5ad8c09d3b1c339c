"""fp64 CPU oracle for the MapFlow hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import or run anything under ``oracle/``.  The product path (the HIP library
and its Python binding) never imports it and shares no code with it.

Every function states the passage of the pages it follows.  Page keys used in citations:

* [MapFlow开源] "MapFlow开源:大模型换班,Prefill为何能快20%?" (aitest123.com), with its sections
  "不传 KV Cache,改传'注意力关系'" (pass attention relations instead of KV),
  "只存重要的:块稀疏压缩" (block-sparse compression) and
  "算得省的:融合内核执行" (fused kernel execution).
* [Reuses Attention] "Peking University's MapFlow Reuses Attention Across Models without
  Recomputing the KV Cache" (roboind.com), sections on the attention map and on the three
  system components.
* [Abstract] "Accelerating Cross-Model LLM Inference via Attention Map Reuse" (weekinpapers.com),
  the abstract.
* [MapFlow 方案] the 52hbtv.com digest, sections 二 (key components).

Parity status: every function here is pinned by tests in ``tests/test_oracle.py`` (brute force,
library routines, closed forms or invariants); none is "parity unpinned".
"""
from .mapflow_oracle import (  # noqa: F401
    OracleBSR,
    attention_rows,
    bf16_round,
    block_masses,
    block_row_compress,
    compress,
    dense_causal_attention,
    apply_v,
    gather_row_probs,
    layer_map,
    mix_heads,
    renormalise,
    retrieve,
    retrieve_layers,
    retrieve_block_row,
    select_blocks,
)
