"""Brute-force DCP slot mapper and local sequence lengths.

Test infrastructure: see the package docstring.

Source: "Decode Context Parallel (DCP)" (vLLM Ascend design doc), section
"KV-cache layout" (the Chinese edition of the same page, section "KV 缓存布局",
states the same four formulas). A virtual block holds ``block_size *
dcp_size`` tokens and for token position ``x``:

    virtual_block_index     = x // (block_size * dcp_size)
    offset_in_virtual_block = x %  (block_size * dcp_size)
    local_block_index       = offset_in_virtual_block // cp_kv_cache_interleave_size
    target_rank             = local_block_index % dcp_size

and the implementation requires ``block_size % cp_kv_cache_interleave_size ==
0``. "DeepSeek V4.1 context parallelism", section "Cache ownership", adds that
writes translate virtual slots to local slots and mask non-owners.

Readings where the pages are silent (each listed in the design notes):

* The page gives the owner of a token but not its offset inside the owner's
  block. Here the owner stores the tokens it owns in ascending position order,
  densely: the offset of token ``x`` is the number of earlier tokens of the
  same virtual block that the same rank owns. It is computed by literally
  running a per-rank counter over one virtual block, not by a closed form.
* The block-table figure is lost. Here one table row per request is indexed by
  ``virtual_block_index`` and is shared by all ranks: every rank keeps its own
  paged pool with identical geometry and the token lands in physical block
  ``block_table[req, virtual_block_index]`` of the owner's pool.
* A non-owner's slot is -1. A negative position, a request index outside the
  table, a virtual block index at or past ``max_vblocks`` or a negative block
  id gives -1 on every rank.
"""

import numpy as np


def target_rank(x, block_size: int, dcp_size: int, interleave: int):
    """The page's four formulas, literally (works on ints and int arrays)."""
    virtual_block_index = x // (block_size * dcp_size)  # noqa: F841 (kept to mirror the page)
    offset_in_virtual_block = x % (block_size * dcp_size)
    local_block_index = offset_in_virtual_block // interleave
    return local_block_index % dcp_size


def _check_args(block_size: int, dcp_size: int, interleave: int):
    if block_size < 1 or dcp_size < 1 or interleave < 1:
        raise ValueError("block_size, dcp_size and interleave must be >= 1")
    if block_size % interleave != 0:
        raise ValueError("block_size % cp_kv_cache_interleave_size must be 0")


def in_block_offsets(block_size: int, dcp_size: int, interleave: int) -> np.ndarray:
    """Offset inside the owner's block for each offset in a virtual block.

    Runs one counter per rank over the ``block_size * dcp_size`` positions of a
    virtual block in ascending order (every virtual block has the same
    pattern, since the formulas see ``x`` only through its offset).
    """
    _check_args(block_size, dcp_size, interleave)
    span = block_size * dcp_size
    counters = [0] * dcp_size
    out = np.empty(span, dtype=np.int64)
    for off in range(span):
        r = int(target_rank(off, block_size, dcp_size, interleave))
        out[off] = counters[r]
        counters[r] += 1
    assert all(c == block_size for c in counters), "constraint violated"
    return out


def slot_mapping(positions, req_indices, block_table, block_size: int,
                 dcp_size: int, interleave: int, max_vblocks: int = None) -> np.ndarray:
    """Slots ``[dcp_size, T]`` (int64); -1 where the rank does not own the token.

    ``positions[T]`` are token positions in their request's sequence,
    ``req_indices[T]`` index rows of ``block_table[num_reqs, max_vblocks]``.
    """
    positions = np.asarray(positions, dtype=np.int64)
    req_indices = np.asarray(req_indices, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    num_reqs = block_table.shape[0]
    if max_vblocks is None:
        max_vblocks = block_table.shape[1]
    offs_in_block = in_block_offsets(block_size, dcp_size, interleave)
    T = positions.shape[0]
    slots = np.full((dcp_size, T), -1, dtype=np.int64)
    for t in range(T):
        x, b = int(positions[t]), int(req_indices[t])
        if x < 0 or b < 0 or b >= num_reqs:
            continue
        vbi = x // (block_size * dcp_size)
        if vbi >= max_vblocks:
            continue
        phys = int(block_table[b, vbi])
        if phys < 0:
            continue
        off = x % (block_size * dcp_size)
        r = int(target_rank(x, block_size, dcp_size, interleave))
        slots[r, t] = phys * block_size + int(offs_in_block[off])
    return slots


def owners(seq_len: int, block_size: int, dcp_size: int, interleave: int) -> np.ndarray:
    """Owner rank of every position ``0..seq_len-1`` (formulas, vectorised)."""
    _check_args(block_size, dcp_size, interleave)
    return target_rank(np.arange(seq_len, dtype=np.int64), block_size, dcp_size, interleave)


def local_positions(seq_len: int, block_size: int, dcp_size: int, interleave: int) -> np.ndarray:
    """Rank-local position of every token: the owner's running count so far."""
    own = owners(seq_len, block_size, dcp_size, interleave)
    out = np.empty(seq_len, dtype=np.int64)
    for r in range(dcp_size):
        idx = np.nonzero(own == r)[0]
        out[idx] = np.arange(idx.shape[0], dtype=np.int64)
    return out


def local_seq_lens(seq_lens, block_size: int, dcp_size: int, interleave: int) -> np.ndarray:
    """``[num_reqs, dcp_size]`` int32: tokens each rank owns (final counter values).

    This is the per-rank context-length matrix of "Decode Context Parallel
    (DCP)", section "Backend structure".
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    out = np.zeros((seq_lens.shape[0], dcp_size), dtype=np.int32)
    for b, L in enumerate(seq_lens):
        if L > 0:
            out[b] = np.bincount(owners(int(L), block_size, dcp_size, interleave),
                                 minlength=dcp_size)
    return out
