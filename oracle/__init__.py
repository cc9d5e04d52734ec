"""Plain, slow CPU oracle for compressed-KV decode attention (numpy, fp64).

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything here. The HIP library and its Python binding never
import it, and it imports nothing from them: the two sides share no code. Only
the seeded input generators in ``workloads/`` feed both.

What it computes, and the page passage each part follows:

* ``quant``     per-token symmetric INT8/INT4 quantize-on-write, dequantize,
                INT4 packing, KV byte accounting ("KV Cache optimization
                techniques" §1.1, §1.2 and "KV Cache的挑战"; "KV Cache
                Compression Report" §3.2)
* ``attention`` softmax(q K^T / sqrt(d)) V over the dequantized cache,
                contiguous and paged (report §1.1 and §3.2; tutorial §3.2)
* ``eviction``  H2O accumulation, sink + recent + top-k keep-set, stable
                compaction (report §3.3, §3.4; tutorial §2.2, §2.4;
                eviction-and-reuse survey §3.3)
* ``cache``     a reference cache and the decode-step schedule
* ``schedule``  per-layer keep budgets, the pyramid schedules (tutorial
                §2.3; eviction-and-reuse survey §4)
* ``blocks``    block-granular H2O eviction on a paged cache (survey §4;
                tutorial §3.2)
* ``tiers``     fp16 sink and recent tiers of a quantized cache (report §3.2;
                tutorial §1.3)
* ``kvsep``     K and V stored apart: scoring on the quantized K, the output
                from the top-k tokens' fp16 V rows (report §3.5)

Floating point is fp64 throughout, except where the method fixes fp32: the
quantization scale and the quotient that is rounded to a code, both taken as
correctly rounded fp32 results.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, brute force on tiny inputs and the values the pages print.
"""
from .attention import attend_head_group, attend_values, decode_attention, paged_decode_attention, paged_gather
from .cache import RefCache, paged_append
from .eviction import compact_row, h2o_accumulate, kth_threshold, select_keep
from .blocks import block_evict, move_block_scores
from .schedule import layer_budgets
from .tiers import tier_bounds, tier_values
from .kvsep import kv_separated_attention
from .quant import (QMAX, QMIN, compressed_bytes_per_token_head, dequantize, kv_bytes_per_token,
                    pack_int4, quantize_rows, unpack_int4)

__all__ = [
    "QMAX", "QMIN", "quantize_rows", "dequantize", "pack_int4", "unpack_int4",
    "kv_bytes_per_token", "compressed_bytes_per_token_head",
    "attend_head_group", "attend_values", "decode_attention", "paged_decode_attention", "paged_gather",
    "h2o_accumulate", "select_keep", "kth_threshold", "compact_row",
    "RefCache", "paged_append", "layer_budgets", "block_evict", "move_block_scores",
    "tier_bounds", "tier_values", "kv_separated_attention",
]
