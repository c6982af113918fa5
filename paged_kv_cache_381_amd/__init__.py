"""MI355X-native paged KV cache and PagedAttention decode.

The compute path lives in ``libpagedkv.so`` (hand-written HIP for gfx950,
C ABI in ``include/pagedkv.h``); this package is its ctypes binding under the
same names plus a small host-side cache object.  There is no fallback: if the
library is not built, loading it raises.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE, PKV_BF16, PKV_F32, PagedKVError, lib, make_layout, pkv_layout,
    pkv_last_error, pkv_version,
    pkv_pool_create, pkv_pool_destroy, pkv_block_alloc, pkv_block_incref, pkv_block_free,
    pkv_block_refcount, pkv_pool_num_free, pkv_seq_create, pkv_seq_fork, pkv_seq_append_slots,
    pkv_batch_append_slots, pkv_seq_free, pkv_seq_len, pkv_seq_block_table, pkv_batch_block_tables,
    pkv_pool_stats, pkv_kv_bytes_per_token, pkv_pool_bytes, pkv_validate_tables,
    paged_kv_append, pkv_copy_blocks, paged_attention_workspace_bytes, paged_attention_decode,
    pkv_decode_plan, paged_attention_plan_bytes, new_decode_plan, reset_decode_plan,
)
