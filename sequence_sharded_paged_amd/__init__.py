"""MI355X-native Decode Context Parallel (DCP) decode attention.

The compute lives in libdcp (HIP, gfx950), reached through the C ABI in
include/dcp.h; ``native`` is the thin ctypes binding with the same function
names, ``cache`` holds the per-rank paged KV pools in the layouts the kernels
read. Importing this package does not load the library; the first call does,
and raises if it has not been built.
"""

from .native import (  # noqa: F401
    DCP_ALGO_AUTO, DCP_ALGO_FAST, DCP_ALGO_GENERIC, DCP_BF16, DCP_F32, DCP_FP8_E4M3, DcpError, KvCache,
    dcp_abi_version, dcp_check_block_table, dcp_gather_context, dcp_kv_cache_write, dcp_local_seq_lens,
    dcp_lse_merge, dcp_partial_decode_attn, dcp_partial_decode_attn_noalloc, DCP_ERR_SCRATCH,
    DCP_NOALLOC_SCRATCH_BYTES,
    dcp_partial_decode_attn_workspace_size, dcp_partial_segment_attn, dcp_partial_segment_attn_workspace_size,
    dcp_partial_verify_attn, dcp_partial_verify_attn_workspace_size,
    dcp_slot_mapping, dcp_status_string, dcp_hbm_read_probe, dcp_hbm_read_probe_blocks,
)
from .cache import PagedKVCache  # noqa: F401
