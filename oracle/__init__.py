"""fp64 CPU oracle for exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).

Every function follows the page titled "把 FlashAttention 搬上昇腾：Triton-Ascend
CV Pipeline 优化实战" ("Porting FlashAttention to Ascend: CV-pipeline
optimisation with Triton-Ascend", BiumBiu, 2026-08-30), cited below as
[FA-Ascend] with the section it comes from; the grouped key/value heads follow
the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu, 2026-04-30), cited
as [Serving-Ascend], as do the variable-length batches and the paged KV cache
(``paged.py``: cache writes and decode attention over pages) and the
query-aware page selection with attention over the selected pages
(``quest.py``); decode attention over two KV sources under one softmax
(``sources.py``) follows the page "在 4 张 A100 上部署 DeepSeek-V4-Flash-0731"
(BiumBiu), section 7.5.

Pinning: every function here is pinned by tests marked ``not gpu`` to facts
other than itself (finite differences, closed forms, invariants, a library
routine, brute force on tiny inputs); see ``tests/test_oracle.py``.  No function
is "parity unpinned".
"""
from .attention import (  # noqa: F401
    attention_forward,
    attention_forward_full,
    attention_backward,
    loss_sum_o_do,
    gqa_kv_head,
    attention_forward_gqa,
    attention_backward_gqa,
    attention_forward_varlen,
    attention_backward_varlen,
)
from .paged import gather_context, paged_decode, reshape_and_cache  # noqa: F401
from .quest import quest_page_minmax, quest_scores, quest_select, quest_sparse_decode  # noqa: F401
from .sources import attention_over_sources, decode_over_sources, source_tokens  # noqa: F401
