"""Reference oracle for paged grouped-query attention: TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU implementation of what the
GPU library computes. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``gqa_paged_kv_amd``) never imports, calls or links it, and
it never imports the product path: the two share no code, headers, tables or
helpers.

Floating point is evaluated in float64 on the exact input values (bf16 and
fp32 inputs widen to float64 without rounding).

Sources, cited by page title and section throughout:

* [TRT-GQA]  "TensorRT对Grouped Query Attention的支持进展"
  (http://www.maplevalley.com.cn/news/471480) -- defines MHA / MQA / GQA
  (section "技术演进背景"), the repeat_kv operation "to match Q" (section
  "图优化与算子融合"), the paged KV pool addressed through physical page
  indices (section "动态形状与KV Cache管理") and the KV-size ratio (section
  "显存带宽瓶颈下的理性妥协").
* [GQA-BATCH] "解锁GQA性能潜力：从批量大小敏感性到高效优化实践"
  (https://blog.gitcode.com/10b38b39ad64e3b8dbe2b300ee340adc.html) -- NumSplits
  (section "核心参数调优：PackGQA与NumSplits的协同舞蹈") and the causal mask
  (caption of Figure 2).
* [TRTLLM-OPS] "TensorRT-LLM与TensorRT核心差异解析", chapter 4 "算子库差异"
  -- the unfused decomposition Q*K^T -> Softmax -> x V (section 4.1), tiling
  that writes only the final result (section 4.2.1) and the page table that
  maps logical to physical pages (section 4.2.2).

Readings taken where the pages are silent (scale 1/sqrt(d), contiguous head
grouping, page layout, split boundaries, partial format) are stated at each
function. Every function here is pinned by tests in ``tests/test_oracle.py``
against brute force, closed forms, a library routine (torch SDPA in float64)
and invariants.
"""

from .fp8 import decode_paged_fp8, dequantize  # noqa: F401
from .attention import (  # noqa: F401
    append_paged,
    append_paged_at,
    combine_splits,
    decode_paged,
    decode_paged_rows,
    decode_split_partials,
    gather_paged,
    kv_bytes,
    kv_head_of,
    logical_to_physical,
    prefill_causal,
    prefill_paged,
    prefill_paged_rows,
    prefill_causal_rows,
    split_page_ranges,
)
