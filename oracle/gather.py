"""Context gather for (chunked) prefill: the inverse of the slot mapping.

Test infrastructure: see the package docstring.

Source: "Decode Context Parallel (DCP)" (vLLM Ascend developer guide), section
"Prefill and chunked prefill": for MLA the context KV cache, spread over the
DCP group, is gathered and put back in request-contiguous order before the
current query chunk attends it; "DeepSeek V4.1 context parallelism", section
"Cache ownership": pages are copied as stored, quantised values included,
without dequantising. Readings taken here:

* request b's context is its positions ``0 .. ctx_lens[b] - 1``; the output
  holds them in request order, then position order, at rows
  ``cu[b] .. cu[b] + ctx_lens[b] - 1`` with ``cu`` the exclusive prefix sum;
* each row is the stored representation (fp32 values, bf16 bits or fp8
  codes) of the position's K row (and V row), copied from the pool of its
  owning rank at the slot the slot mapping gives;
* a position the block table does not map (negative block id, virtual block
  past ``max_vblocks``) yields a zero row.
"""

import numpy as np

from . import layout


def gather_context(k_pool, v_pool, block_table, ctx_lens, block_size: int, dcp_size: int, interleave: int,
                   max_vblocks: int = None):
    """``k_pool [R, N, H, bs, Dk]`` (stored), ``v_pool [R, N, H, Dv, bs]`` or
    None, ``block_table [B, W]``, ``ctx_lens [B]`` -> ``(K [T, H, Dk],
    V [T, H, Dv] or None)`` with ``T = sum(ctx_lens)``."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    B = ctx_lens.shape[0]
    positions = np.concatenate([np.arange(n, dtype=np.int64) for n in ctx_lens] + [np.zeros(0, np.int64)])
    reqs = np.concatenate([np.full(n, b, dtype=np.int64) for b, n in enumerate(ctx_lens)] + [np.zeros(0, np.int64)])
    slots = layout.slot_mapping(positions, reqs, block_table, block_size, dcp_size, interleave, max_vblocks)
    T, H, Dk = positions.shape[0], k_pool.shape[2], k_pool.shape[4]
    out_k = np.zeros((T, H, Dk), dtype=k_pool.dtype)
    out_v = None if v_pool is None else np.zeros((T, H, v_pool.shape[3]), dtype=v_pool.dtype)
    for t in range(T):
        for r in range(dcp_size):
            s = int(slots[r, t])
            if s < 0:
                continue
            blk, off = divmod(s, block_size)
            out_k[t] = k_pool[r, blk, :, off, :]
            if out_v is not None:
                out_v[t] = v_pool[r, blk, :, :, off]
    return out_k, out_v
