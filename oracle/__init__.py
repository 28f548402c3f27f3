"""CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The library itself (``paged_kv_cache_186_amd``) never imports
it and has no CPU fallback: its kernels are the only compute path.

The oracle is a plain, slow, obviously correct restatement of what the method
computes, in float64, written with numpy (plus torch CPU indexing where a
storage dtype such as bfloat16 has no numpy equivalent).  It shares no code,
constants or helpers with the HIP kernels.

Sources, cited by page title and section:

* vLLM tutorial page "3. PagedAttention原理" (chapter 3 of a Chinese guide to
  long-sequence memory optimisation in vLLM): §3.2 (logical KV blocks mapped to
  scattered physical blocks through a page table), §3.3.1 (block size 16 or 32),
  §3.3.2 (on-demand allocation, one new block when the last is full),
  §3.3.3 (shared blocks with reference counts), §3.4 closing remarks (paging
  changes memory management only, not the mathematics of attention).
* Page "PagedAttentionMetal：基于Metal 3的Apple Silicon原生LLM推理加速方案",
  sections 块表管理 (block table: logical→physical, copying and sharing of
  blocks) and 注意力计算优化 (attention reads K/V through the block table;
  variable-length batches without padding).
* Page "mlx-paged-attention: Bringing vLLM-level High Throughput Inference to
  Apple Silicon", core feature 2 (shared prefixes with copy-on-write).
* Page "PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎",
  architecture list (the kernel gathers K/V from the physical pool),
  roadmap milestone 3 (multi-head latent attention, ``oracle.multi_query``)
  and milestone 4 (the name "Flash-Dec", the only hint of a split-context
  decode on the pages).
* Page "mlx-paged-attention: ...", comparison with vLLM and future plans
  (speculative decoding: several new query tokens per sequence,
  ``oracle.multi_query``).

Pins: every function here is checked in ``tests/test_oracle.py`` against facts
that do not come from the oracle itself (hand-derived fixtures under
``tests/golden/``, closed forms, a library attention routine, invariants).
Parity status per function is listed in the module docstring of
``oracle.paged_attention``.
"""

from .paged_attention import (  # noqa: F401
    gather_sequence_kv,
    decode_ref,
    split_decode_ref,
    lse_merge_ref,
    reshape_and_cache_ref,
    copy_blocks_ref,
    swap_blocks_ref,
    decode_gqa_ref,
)
from .multi_query import (  # noqa: F401
    prefill_ref,
    mla_decode_ref,
)
from .fp8 import (  # noqa: F401
    fp8_values,
    quantize_fp8_ref,
    dequant_ref,
    decode_fp8_ref,
    reshape_and_cache_fp8_ref,
    copy_blocks_fp8_ref,
)
