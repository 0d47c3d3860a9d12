"""Shared test plumbing: device inputs for the HIP path, oracle evaluation on
the host, and the parity checks (tolerances from the project's acceptance
bar: max-abs 1e-5 for fp32 and 2e-2 for bf16/fp8 inputs, plus a per-row
relative bound and an LSE bound so that long rows, whose outputs are small,
cannot pass vacuously)."""

import numpy as np
import torch

import sequence_sharded_paged_amd as dcp
from workloads.generate import stored_numpy, stored_format


def _oracle():
    """The oracle modules, imported only by the functions that check against
    them: the device-side set-up below (DeviceInputs, VerifyRun,
    SegmentInputs), which bench.py also uses, never loads the oracle."""
    from oracle import attention, formats, layout
    return attention, formats, layout

TOL = {
    "fp32": dict(max_abs=1e-5, row_rel=1e-4, lse=1e-5),
    "bf16": dict(max_abs=2e-2, row_rel=1e-2, lse=1e-3),
    "fp8_e4m3": dict(max_abs=2e-2, row_rel=1e-2, lse=1e-3),
}
OUT_BF16_EXTRA = 2.0 ** -8   # relative rounding of a bf16 output element


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
            self.cache.write(slots, case.k[b].to(device), None if case.v is None else case.v[b].to(device))
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


def oracle_request(case, b, dcp_size=None, interleave=None, with_partials=True):
    """Float64 oracle for request b: full attention (with the sink) and the
    per-rank partials over the brute-force ownership."""
    oatt, ofmt, olay = _oracle()
    w = case.workload
    D = dcp_size or w.dcp_size
    I = interleave or w.interleave
    q = ofmt.decode(stored_numpy(case.q[b]), stored_format(case.q))
    k = ofmt.decode_kv(stored_numpy(case.k[b]), stored_format(case.k[b]), case.k_scale)
    if case.v is None:
        v = k[:, :, :w.head_dim_v]
    else:
        v = ofmt.decode_kv(stored_numpy(case.v[b]), stored_format(case.v[b]), case.v_scale)
    full = oatt.decode_attention(q, k, v, w.softmax_scale, case.sink)
    parts = None
    if with_partials:
        own = olay.owners(int(case.seq_lens[b]), w.block_size, D, I)
        parts = oatt.rank_partials(q, k, v, w.softmax_scale, own, D)
    return full, parts


def check_rows(got, ref, tol, what, out_bf16=False):
    """Element-wise max-abs and per-row relative bounds for [H, Dv] outputs."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = tol["max_abs"]
    assert err.max() <= max_abs, f"{what}: max-abs {err.max():.3e} > {max_abs}"
    rel_tol = tol["row_rel"] + (OUT_BF16_EXTRA if out_bf16 else 0.0)
    row_ref = np.maximum(np.abs(ref).max(axis=-1), 1e-3)
    rel = err.max(axis=-1) / row_ref
    assert rel.max() <= rel_tol, f"{what}: row-relative {rel.max():.3e} > {rel_tol}"


def check_lse(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf pattern differs"
    d = np.abs(got[~inf_ref] - ref[~inf_ref])
    if d.size:
        assert d.max() <= tol["lse"], f"{what}: LSE err {d.max():.3e} > {tol['lse']}"


def check_against_oracle(inputs, result, requests=None, check_parts=True, rank_begin=0):
    case, w = inputs.case, inputs.w
    po, pl, o, lse = [t.float().cpu().numpy() for t in result]
    tol = TOL[w.kv_format]
    R = po.shape[0]
    for b in (range(case.batch) if requests is None else requests):
        (fo, fl), parts = oracle_request(case, b, inputs.D, inputs.I, with_partials=check_parts)
        if R == inputs.D:
            check_rows(o[b], fo, tol, f"merged O b={b}", out_bf16=(w.out_format == "bf16"))
            check_lse(lse[b], fl, tol, f"merged LSE b={b}")
        if check_parts:
            ro, rl = parts
            for r in range(R):
                check_rows(po[r, b], ro[rank_begin + r], tol, f"partial O r={rank_begin + r} b={b}")
                check_lse(pl[r, b], rl[rank_begin + r], tol, f"partial LSE r={rank_begin + r} b={b}")


# ---------------------------------------------------------------------------
# multi-token decode (speculative verification)
# ---------------------------------------------------------------------------
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


def oracle_verify_request(case, q, b, dcp_size, interleave):
    """Float64 oracle for request b's q_len query tokens: causal attention over
    the cached sequence (with the sink) and the per-rank partials."""
    oatt, ofmt, olay = _oracle()
    w = case.workload
    qb = ofmt.decode(stored_numpy(q[b]), stored_format(q))                     # [q_len, Hq, Dk]
    k = ofmt.decode_kv(stored_numpy(case.k[b]), stored_format(case.k[b]), case.k_scale)
    v = k[:, :, :w.head_dim_v] if case.v is None else ofmt.decode_kv(stored_numpy(case.v[b]),
                                                                      stored_format(case.v[b]), case.v_scale)
    full = oatt.verify_attention(qb, k, v, w.softmax_scale, case.sink)
    own = olay.owners(int(case.seq_lens[b]), w.block_size, dcp_size, interleave)
    parts = oatt.verify_rank_partials(qb, k, v, w.softmax_scale, own, dcp_size)
    return full, parts


def check_verify_against_oracle(run, result, requests=None, check_parts=True):
    inputs = run.inputs
    case, w = inputs.case, inputs.w
    po, pl, o, lse = [t.float().cpu().numpy() for t in result]
    tol = TOL[w.kv_format]
    R = po.shape[0]
    for b in (range(case.batch) if requests is None else requests):
        (fo, fl), (ro, rl) = oracle_verify_request(case, run.q.cpu(), b, inputs.D, inputs.I)
        for i in range(run.q_len):
            if R == inputs.D:
                check_rows(o[b, i], fo[i], tol, f"merged O b={b} i={i}", out_bf16=(w.out_format == "bf16"))
                check_lse(lse[b, i], fl[i], tol, f"merged LSE b={b} i={i}")
            if check_parts:
                for r in range(R):
                    rr = run.rank_begin + r
                    check_rows(po[r, b, i], ro[rr, i], tol, f"partial O r={rr} b={b} i={i}")
                    check_lse(pl[r, b, i], rl[rr, i], tol, f"partial LSE r={rr} b={b} i={i}")


# ---------------------------------------------------------------------------
# replicated segment (a sliding-window cache counted by one rank)
# ---------------------------------------------------------------------------
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
            self.cache.write(slots, seg.k[b].to(device), None if seg.v is None else seg.v[b].to(device))
        self.kv = self.cache.descriptor(0)
        B, Hq = inputs.q.shape[0], inputs.q.shape[1]
        n = dcp.dcp_partial_segment_attn_workspace_size(B, Hq, dcp.native.TORCH_TO_DCP[inputs.q.dtype], self.kv)
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    def fold(self, seg_rank, algo=dcp.DCP_ALGO_AUTO):
        i = self.inputs
        dcp.dcp_partial_segment_attn(i.q, self.kv, self.block_table, self.lens, i.w.softmax_scale, seg_rank,
                                     i.rank_begin, i.rank_count, i.po, i.pl, self.ws, algo=algo)


def oracle_segment_request(case, seg, b, dcp_size, interleave, seg_rank):
    """Float64 oracle for request b with its segment: attention over the
    sequence and the segment together (sink included) and the per-rank
    partials with the segment on rank seg_rank."""
    oatt, ofmt, olay = _oracle()
    w = case.workload
    q = ofmt.decode(stored_numpy(case.q[b]), stored_format(case.q))

    def kv(kt, vt):
        k = ofmt.decode_kv(stored_numpy(kt), stored_format(kt), case.k_scale)
        v = k[:, :, :w.head_dim_v] if vt is None else ofmt.decode_kv(stored_numpy(vt), stored_format(vt),
                                                                      case.v_scale)
        return k, v

    k, v = kv(case.k[b], None if case.v is None else case.v[b])
    ks, vs = kv(seg.k[b], None if seg.v is None else seg.v[b])
    full = oatt.decode_attention(q, np.concatenate([k, ks]), np.concatenate([v, vs]), w.softmax_scale, case.sink)
    own = olay.owners(int(case.seq_lens[b]), w.block_size, dcp_size, interleave)
    parts = oatt.segment_rank_partials(q, k, v, w.softmax_scale, own, dcp_size, ks, vs, seg_rank)
    return full, parts


def check_segment_against_oracle(inputs, seg, seg_rank, result, requests=None):
    case, w = inputs.case, inputs.w
    po, pl, o, lse = [t.float().cpu().numpy() for t in result]
    tol = TOL[w.kv_format]
    R = po.shape[0]
    for b in (range(case.batch) if requests is None else requests):
        (fo, fl), (ro, rl) = oracle_segment_request(case, seg, b, inputs.D, inputs.I, seg_rank)
        if R == inputs.D:
            check_rows(o[b], fo, tol, f"merged O b={b}", out_bf16=(w.out_format == "bf16"))
            check_lse(lse[b], fl, tol, f"merged LSE b={b}")
        for r in range(R):
            rr = inputs.rank_begin + r
            check_rows(po[r, b], ro[rr], tol, f"partial O r={rr} b={b}")
            check_lse(pl[r, b], rl[rr], tol, f"partial LSE r={rr} b={b}")
