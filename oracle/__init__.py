"""CPU oracle for the paged KV-cache write and paged attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and never falls back to it.

Everything here is plain, slow and written to be checked by eye against the
source pages; floating point is evaluated in float64.  The pages are cited by
title and section:

* HB  - inference-systems handbook, chapter "分页 KV Cache" (Paged KV Cache),
        anrans.github.io
* XQ  - xxqk.cn article summarising vLLM PagedAttention (SOSP 2023) with a toy
        simulator
* MV  - mini-vllm tutorial step 12, "PagedAttention：分页内存管理"
* KC  - "KV cache：容量推导、分页与回收" (capacity, paging, reclamation),
        blog.mlxb.cc
* AQ  - aiqz.cc article "paged-attention"
"""

from .paged_attention import (  # noqa: F401
    copy_blocks,
    swap_blocks,
    widen,
    slot_for,
    slot_mapping,
    num_blocks,
    tail_slots,
    reshape_and_cache,
    gather,
    paged_attention,
    decode_attention,
    contiguous_attention,
    brute_force_decode,
)
from .capacity import kv_bytes, kv_bytes_per_token, paged_utilisation  # noqa: F401
from .layout import convert_blocks, fuse_kv, reshape_and_cache_fused, split_kv  # noqa: F401
