"""Device-resident inputs for the HIP path, built from a generated case.

This is set-up, not the method: the per-rank pools are allocated in the
layouts the kernels read, the canonical rows are placed at the slots the
library's own slot mapping returns (a torch scatter of stored bits), and the
calls of one decode, verification or segment step are bound to those
buffers, so that ``step()`` launches without allocating. bench.py times
through these classes and the GPU tests use them; they import nothing from
the oracle.
"""

import numpy as np
import torch

import sequence_sharded_paged_amd as dcp


def _raw(t):
    """Integer view of the same bytes (index_put is not implemented for fp8)."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def scatter_rows(cache, slots, k_rows, v_rows=None):
    """Place canonical rows ``k_rows [T, Hkv, Dk]`` (and ``v_rows``) of a
    ``PagedKVCache`` at ``slots [num_ranks, T]`` (-1 = not on that rank),
    copying the stored bits. Test and benchmark set-up only: the library's
    kernel for this step (with quantisation) is ``dcp_kv_cache_write``."""
    bs = cache.block_size
    kraw, kin = _raw(cache.k), _raw(k_rows)
    vraw = None if cache.v is None else _raw(cache.v)
    vin = None if v_rows is None else _raw(v_rows)
    for r in range(cache.num_ranks):
        sel = slots[r] >= 0
        s = slots[r][sel]
        if s.numel() == 0:
            continue
        blk, off = s // bs, s % bs
        kraw[r][blk, :, off, :] = kin[sel]
        if vraw is not None:
            if cache.v_layout == "dim_major":
                vraw[r][blk, :, :, off] = vin[sel]
            else:
                vraw[r][blk, :, off, :] = vin[sel]


class DeviceInputs:
    """Everything the HIP path reads, built from a generated ``Case``."""

    def __init__(self, case, device="cuda", dcp_size=None, interleave=None, v_layout="dim_major",
                 fill="nan"):
        w = case.workload
        self.case, self.w = case, w
        self.D = dcp_size or w.dcp_size
        self.I = interleave or w.interleave
        self.bs = w.block_size
        lens = case.seq_lens
        if dcp_size is not None or interleave is not None:
            span = self.bs * self.D
            nvb = [(int(L) + span - 1) // span for L in lens]
            rng = np.random.default_rng(1234)
            nblk = max(1, sum(nvb))
            perm = rng.permutation(nblk).astype(np.int32)
            table = np.full((len(lens), max(nvb + [1])), -1, dtype=np.int32)
            pos = 0
            for b, n in enumerate(nvb):
                table[b, :n] = perm[pos:pos + n]
                pos += n
        else:
            table, nblk = case.block_table, case.num_blocks
        self.block_table_np = table
        self.block_table = torch.from_numpy(table).to(device)
        self.seq_lens = torch.from_numpy(lens.astype(np.int32)).to(device)
        self.local_lens = dcp.dcp_local_seq_lens(self.seq_lens, self.bs, self.D, self.I)
        self.q = case.q.to(device)
        kv_dtype = case.k[0].dtype
        self.cache = dcp.PagedKVCache(self.D, nblk, self.bs, w.num_kv_heads, w.head_dim_k, w.head_dim_v,
                                      kv_dtype, mla=w.mla, device=device, v_layout=v_layout,
                                      k_scale=case.k_scale, v_scale=case.v_scale, fill=fill)
        for b in range(case.batch):
            L = int(lens[b])
            if L == 0:
                continue
            pos = torch.arange(L, dtype=torch.int64, device=device)
            req = torch.full((L,), b, dtype=torch.int32, device=device)
            slots = dcp.dcp_slot_mapping(pos, req, self.block_table, self.bs, self.D, self.I)
            scatter_rows(self.cache, slots, case.k[b].to(device), None if case.v is None else case.v[b].to(device))
        self.sink = None if case.sink is None else torch.from_numpy(case.sink).to(device)
        torch.cuda.synchronize()

    def prepare(self, algo=dcp.DCP_ALGO_AUTO, rank_begin=0, rank_count=None, out_dtype=None):
        """Allocate workspace and outputs once (NaN-filled so unwritten
        entries show up); ``step`` then launches without allocating."""
        w = self.w
        R = self.D - rank_begin if rank_count is None else rank_count
        B, Hq = self.q.shape[0], self.q.shape[1]
        dev = self.q.device
        self.algo, self.rank_begin, self.rank_count = algo, rank_begin, R
        self.kv = self.cache.descriptor(rank_begin)
        ws_bytes = dcp.dcp_partial_decode_attn_workspace_size(B, Hq, dcp.native.TORCH_TO_DCP[self.q.dtype],
                                                              self.kv, R, algo)
        self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.po = torch.full((R, B, Hq, w.head_dim_v), float("nan"), dtype=torch.float32, device=dev)
        self.pl = torch.full((R, B, Hq), float("nan"), dtype=torch.float32, device=dev)
        od = {"bf16": torch.bfloat16, "fp32": torch.float32}[out_dtype or w.out_format]
        self.o = torch.full((B, Hq, w.head_dim_v), float("nan"), dtype=od, device=dev)
        self.lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
        return self

    def partial(self):
        dcp.dcp_partial_decode_attn(self.q, self.kv, self.block_table, self.local_lens, self.D, self.rank_begin,
                                    self.rank_count, self.w.softmax_scale, self.po, self.pl, self.ws,
                                    algo=self.algo)

    def merge(self):
        dcp.dcp_lse_merge(self.po, self.pl, sink=self.sink, out_o=self.o, out_lse=self.lse)

    def step(self):
        """One decode step: every rank's partial attention, then the merge."""
        self.partial()
        self.merge()

    def run(self, algo=dcp.DCP_ALGO_AUTO, rank_begin=0, rank_count=None, out_dtype=None):
        self.prepare(algo, rank_begin, rank_count, out_dtype)
        self.step()
        torch.cuda.synchronize()
        return self.po, self.pl, self.o, self.lse


def verify_query_lens(seq_lens, q_len):
    """[B, q_len] sequence lengths each query token sees: L_b - q_len + i + 1."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return (lens[:, None] - q_len + np.arange(q_len)[None, :] + 1).astype(np.int32)


class VerifyRun:
    """The HIP path of one multi-token decode step over DeviceInputs' cache:
    per-query local lengths (dcp_local_seq_lens), every rank's partials
    (dcp_partial_verify_attn) and the merge over batch * q_len rows."""

    def __init__(self, inputs, q, algo=dcp.DCP_ALGO_AUTO, rank_begin=0, rank_count=None):
        self.inputs, self.q, self.algo = inputs, q, algo
        w, dev = inputs.w, q.device
        B, self.q_len, Hq, _ = q.shape
        self.rank_begin = rank_begin
        self.R = R = inputs.D - rank_begin if rank_count is None else rank_count
        ql = verify_query_lens(inputs.case.seq_lens, self.q_len)
        assert (ql >= 1).all(), "every queried token must be in the cache"
        self.local_lens = dcp.dcp_local_seq_lens(torch.from_numpy(ql.reshape(-1)).to(dev), inputs.bs, inputs.D,
                                                 inputs.I).view(B, self.q_len, inputs.D)
        self.kv = inputs.cache.descriptor(rank_begin)
        ws_bytes = dcp.dcp_partial_verify_attn_workspace_size(B, self.q_len, Hq, dcp.native.TORCH_TO_DCP[q.dtype],
                                                              self.kv, R, algo)
        self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.po = torch.full((R, B, self.q_len, Hq, w.head_dim_v), float("nan"), dtype=torch.float32, device=dev)
        self.pl = torch.full((R, B, self.q_len, Hq), float("nan"), dtype=torch.float32, device=dev)
        od = {"bf16": torch.bfloat16, "fp32": torch.float32}[w.out_format]
        self.o = torch.full((B * self.q_len, Hq, w.head_dim_v), float("nan"), dtype=od, device=dev)
        self.lse = torch.full((B * self.q_len, Hq), float("nan"), dtype=torch.float32, device=dev)

    def partial(self):
        dcp.dcp_partial_verify_attn(self.q, self.kv, self.inputs.block_table, self.local_lens, self.inputs.D,
                                    self.rank_begin, self.R, self.inputs.w.softmax_scale, self.po, self.pl, self.ws,
                                    algo=self.algo)

    def merge(self):
        B, Hq, Dv = self.q.shape[0], self.q.shape[2], self.inputs.w.head_dim_v
        dcp.dcp_lse_merge(self.po.view(self.R, B * self.q_len, Hq, Dv), self.pl.view(self.R, B * self.q_len, Hq),
                          sink=self.inputs.sink, out_o=self.o, out_lse=self.lse)

    def step(self):
        self.partial()
        self.merge()

    def run(self):
        self.step()
        torch.cuda.synchronize()
        B, Hq, Dv = self.q.shape[0], self.q.shape[2], self.inputs.w.head_dim_v
        return (self.po, self.pl, self.o.view(B, self.q_len, Hq, Dv), self.lse.view(B, self.q_len, Hq))


class SegmentInputs:
    """A generated Segment in device memory: a one-rank pool of the cache's
    geometry (NaN-filled), its block table and lengths, and the call that
    folds it into one rank's partial."""

    def __init__(self, inputs, seg, device="cuda"):
        w = inputs.w
        self.inputs, self.seg = inputs, seg
        self.lens = torch.from_numpy(seg.lens).to(device)
        self.block_table = torch.from_numpy(seg.block_table).to(device)
        self.cache = dcp.PagedKVCache(1, seg.num_blocks, w.block_size, w.num_kv_heads, w.head_dim_k, w.head_dim_v,
                                      inputs.cache.dtype, mla=w.mla, device=device,
                                      k_scale=inputs.case.k_scale, v_scale=inputs.case.v_scale, fill="nan")
        for b in range(len(seg.lens)):
            L = int(seg.lens[b])
            if L == 0:
                continue
            pos = torch.arange(L, dtype=torch.int64, device=device)
            req = torch.full((L,), b, dtype=torch.int32, device=device)
            slots = dcp.dcp_slot_mapping(pos, req, self.block_table, w.block_size, 1, 1)
            scatter_rows(self.cache, slots, seg.k[b].to(device), None if seg.v is None else seg.v[b].to(device))
        self.kv = self.cache.descriptor(0)
        B, Hq = inputs.q.shape[0], inputs.q.shape[1]
        n = dcp.dcp_partial_segment_attn_workspace_size(B, Hq, dcp.native.TORCH_TO_DCP[inputs.q.dtype], self.kv)
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    def fold(self, seg_rank, algo=dcp.DCP_ALGO_AUTO):
        i = self.inputs
        dcp.dcp_partial_segment_attn(i.q, self.kv, self.block_table, self.lens, i.w.softmax_scale, seg_rank,
                                     i.rank_begin, i.rank_count, i.po, i.pl, self.ws, algo=algo)
