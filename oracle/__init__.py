"""CPU oracle for paged-KV attention: test infrastructure only (tests, smoke check, CPU baseline)."""
from .paged_attention import (  # noqa: F401
    attend, causal_key_count, copy_blocks, decode, decode_partitioned, decode_shared_prefix, exact_scale, gather, gather_fast,
    kv_head_of, kv_write, lse_merge, max_abs_err, max_rownorm_rel_err, partition_partials,
    prefill_chunk, slot_location, to_f64, token_location,
)
from . import fp8_cache  # noqa: F401,E402
