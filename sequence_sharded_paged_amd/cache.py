"""Per-rank paged KV pools in the layouts the libdcp kernels read.

Each of ``num_ranks`` ranks owns a pool of ``num_blocks`` physical blocks with
identical geometry; one block-table row per request, indexed by virtual block,
is shared by all ranks (physical id p means block p of the owning rank's
pool). Layouts:

* K: ``[rank, block, kv_head, token, dim]`` (dim contiguous);
* V (GQA): ``[rank, block, kv_head, dim, token]`` (token contiguous, "V
  transposed inside a block"), which the MFMA kernel loads straight into its
  operand layout; ``v_layout="token_major"`` gives ``[..., token, dim]`` for
  the generic kernel;
* MLA: no V tensor; the value is the first ``head_dim_v`` entries of the K
  row (one latent vector serves as key and value).

The pools are filled by ``dcp_kv_cache_write`` (new rows quantised to the
pool format at the slots ``dcp_slot_mapping`` produced).
"""

import torch

from . import native


class PagedKVCache:
    def __init__(self, num_ranks, num_blocks, block_size, num_kv_heads, head_dim_k, head_dim_v,
                 dtype, mla=False, device="cuda", v_layout="dim_major", k_scale=None, v_scale=None,
                 fill=None):
        self.num_ranks, self.num_blocks, self.block_size = num_ranks, num_blocks, block_size
        self.num_kv_heads, self.head_dim_k, self.head_dim_v = num_kv_heads, head_dim_k, head_dim_v
        self.dtype, self.mla, self.v_layout = dtype, mla, v_layout
        R, N, H, bs = num_ranks, num_blocks, num_kv_heads, block_size
        self.k = self._alloc((R, N, H, bs, head_dim_k), dtype, device, fill)
        if mla:
            self.v = None
        elif v_layout == "dim_major":
            self.v = self._alloc((R, N, H, head_dim_v, bs), dtype, device, fill)
        elif v_layout == "token_major":
            self.v = self._alloc((R, N, H, bs, head_dim_v), dtype, device, fill)
        else:
            raise ValueError(v_layout)
        self.k_scale = None if k_scale is None else torch.as_tensor(k_scale, dtype=torch.float32, device=device)
        self.v_scale = None if v_scale is None else torch.as_tensor(v_scale, dtype=torch.float32, device=device)
        if mla and self.k_scale is not None and self.v_scale is None:
            self.v_scale = self.k_scale

    @staticmethod
    def _alloc(shape, dtype, device, fill):
        t = torch.empty(shape, dtype=dtype, device=device)
        raw = _raw(t)
        if fill == "nan":      # a NaN bit pattern: any read of an unwritten slot poisons the result
            raw.fill_({1: 0x7F, 2: 0x7FC0, 4: 0x7FC00000}[t.element_size()])
        else:
            raw.zero_()
        return t

    def descriptor(self, rank_begin=0) -> native.KvCache:
        """``dcp_kv_cache_t`` for ranks ``rank_begin..`` of these pools."""
        d = native.KvCache()
        d.dtype = native.TORCH_TO_DCP[self.dtype]
        d.num_blocks, d.block_size, d.num_kv_heads = self.num_blocks, self.block_size, self.num_kv_heads
        d.head_dim_k, d.head_dim_v = self.head_dim_k, self.head_dim_v
        kr = self.k[rank_begin]
        d.k = kr.data_ptr()
        for i, s in enumerate(self.k.stride()):
            d.k_stride[i] = s
        if self.v is None:
            d.v = None
        else:
            d.v = self.v[rank_begin].data_ptr()
            st = self.v.stride()
            if self.v_layout == "dim_major":   # [rank, block, head, dim, token] -> (rank, block, head, token, dim)
                st = (st[0], st[1], st[2], st[4], st[3])
            for i, s in enumerate(st):
                d.v_stride[i] = s
        d.k_scale = None if self.k_scale is None else self.k_scale.data_ptr()
        d.v_scale = None if self.v_scale is None else self.v_scale.data_ptr()
        return d


def _raw(t):
    """Integer view of the same bytes (index_put is not implemented for fp8)."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])
