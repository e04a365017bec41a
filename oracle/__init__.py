"""fp64 CPU oracle for paged single-token decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code, header, table or helper with the HIP library; both sides are
fed by the seeded generators in ``synth``, which hold none of the method's
arithmetic.

The oracle is written from five web pages on KV caches and PagedAttention.
Citations name a page by its site and give the section heading, equation or
table on that page:

  faulkner  -- "LLM 推理底层：KV Cache 显存几何、GQA/MLA 压缩与 PagedAttention 调度"
               (blog.faulkner.fun/posts/llm-kv-cache-and-paged-attention)
  qwbw      -- "【infra之路】10-PagedAttention 与 KV Cache 管理"
               (www.qwbw.cn/news/28817), numbered sections 1.1 ... 8
  guijiagi  -- KV cache guide (guijiagi.com/posts/kv-cache-guide/),
               numbered sections 1 ... 8
  talentme  -- "KV Cache 显存管理全景 ..." (talentme.airsota.com/.../kv-cache-and-paged-attention)
  hx        -- "LLM 推理引擎设计：KV Cache、PagedAttention 与连续批处理"
               (hx.sn.cn/archives/llm-inference-engine)

Every function here is pinned by ``-m "not gpu"`` tests against closed
forms, worked examples printed on the pages, brute force in exact decimal
arithmetic and library special cases (see ``tests/test_oracle_*.py``).
"""

from .paged_attention import (  # noqa: F401
    widen,
    bf16_bits_to_f64,
    logical_position,
    slot_of,
    slot_mapping,
    reshape_and_cache,
    gather_sequence,
    softmax_weights,
    decode_attention_contiguous,
    window_start,
    paged_decode_attention,
    quantize_int8_rows,
    dequantize_int8,
    paged_decode_attention_int8,
    quantize_int4_rows,
    pack_int4,
    unpack_int4,
    paged_decode_attention_int4,
    paged_prefill_attention,
    paged_decode_attention_mla,
    split_partials,
    merge_partials,
    kv_cache_bytes,
    decode_attention_intensity,
)
from .block_allocator import (  # noqa: F401
    block_hash,
    BlockAllocator,
    copy_blocks,
    swap_out,
    swap_in,
)
