"""CPU oracle for paged decode attention and the paged cache write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library under ``paged_kv_decode_attention_amd/`` and imports nothing
from it; both sides receive the same seeded input arrays and nothing else.

Everything is plain NumPy in float64.  Each function cites the passage of the
source pages it follows:

* "MiniPaged-Qwen: 把 Paged Attention 讲清楚" (blog.zsmgc.love), written
  [MiniPaged-Qwen §x] below -- the authority on what is computed;
* "PagedAttention 源码解析: KV Cache 怎么管理" (jsqmd.com), [PA-source §x];
* "vLLM 与 PagedAttention: 把 KV Cache 变成分页状态" (wineandchord.com),
  [vLLM-paging "section"];
* "2.1 KV Cache 与 PagedAttention 原理" (aiknowledge.cn), [KV-principles §x].

Parity status: every function here is pinned by ``tests/test_oracle.py``
(closed forms, invariants, brute force, a library special case and the
worked examples the pages print) or, for the block pool and the block copy
(``block_pool.py``), by ``tests/test_block_pool_oracle.py`` (the printed
copy-on-write example and invariants), or, for the FP8 KV cache
(``fp8.py``), by ``tests/test_fp8_oracle.py`` (the E4M3 definition,
PyTorch's float8_e4m3fn cast where it is defined, exhaustive round trips,
ties and saturation), or, for the INT8 KV cache (``int8.py``), by
``tests/test_int8_oracle.py`` (two's complement codes, exhaustive round
trips, torch.round's ties-to-even over every bf16 bit pattern, brute-force
nearest integers, saturation); none is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    NEG_INF,
    num_logical_blocks,
    tail_waste,
    kv_head_of,
    gather_sequence_kv,
    decode_contiguous,
    decode_online,
    decode_partitioned,
    decode_verify,
    partition_state,
    lse_merge,
    reshape_and_cache,
    kv_cache_bytes,
    kv_cache_bytes_hidden_form,
)
from .block_pool import BlockPool, PoolExhausted, copy_blocks  # noqa: F401,E402
from . import fp8  # noqa: F401,E402
