"""Decode, verification and segment steps captured once in a HIP graph at a
fixed capacity (batch, block-table width, pools) and replayed while the
lengths change in place, every replay checked against the oracle.

Between replays the test overwrites, in device memory the graph reads:
the sequence lengths (the captured step recomputes the per-rank lengths from
them with dcp_local_seq_lens), the block-table entries (a request that grows
into a new virtual block gets its entry only then; entries past a request's
length hold -1) and, for the segment step, the segment lengths. The length
sets grow requests by one token, cross a virtual-block boundary, take a
request (and with it rank 0's shard) from empty to one token, shrink requests,
empty one request and then all of them. This is the graph-safety property the
"DeepSeek V4.1 context parallelism" note asks of decode metadata (section
"Decode computation": static capacity bounds; section "Validation and
tradeoffs": repeated graph replay with changing lengths): grids and
workspaces depend on the capacity only, and every length is read on the
device.
"""

import dataclasses

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from tests.harness import check_against_oracle, check_segment_against_oracle, check_verify_against_oracle
from workloads import get_workload, make_case, make_segment, make_verify_queries
from workloads.device import DeviceInputs, SegmentInputs, VerifyRun, verify_query_lens

pytestmark = pytest.mark.gpu

# capacity per request and the length sets replayed (bs 64, dcp 8: a virtual block spans 512 positions)
CAP = [1500, 1030, 600, 70]
DECODE_SETS = [
    [1000, 512, 0, 70],       # the set at capture
    [1001, 513, 1, 70],       # +1 token; request 1 enters virtual block 1; request 2 empty -> one token
    [1500, 1030, 600, 0],     # capacity; request 3 empty
    [64, 1, 65, 69],          # shrink; request 2 spills one token past the first interleave chunk
    [0, 0, 0, 0],             # every request empty
    [999, 1029, 599, 1],
]
VERIFY_SETS = [  # every queried token must be cached: L >= q_len
    [1000, 512, 2, 70],
    [1001, 513, 3, 70],
    [1500, 1030, 600, 2],
    [64, 2, 65, 69],
    [999, 1029, 599, 2],
]


def _table_for(cap_table, lens, span):
    """The capacity table with the entries past each request's length set to -1."""
    t = np.full_like(cap_table, -1)
    for b, L in enumerate(lens):
        n = (int(L) + span - 1) // span
        t[b, :n] = cap_table[b, :n]
    return t


def _truncated(case, lens):
    """The case as the oracle sees it at these lengths: each request's first L
    cached rows (positions 0 .. L - 1 hold the same rows at every length)."""
    lens = np.asarray(lens, dtype=np.int32)
    k = [case.k[b][:int(L)] for b, L in enumerate(lens)]
    v = None if case.v is None else [case.v[b][:int(L)] for b, L in enumerate(lens)]
    return dataclasses.replace(case, seq_lens=lens, k=k, v=v)


class _View:
    """What the oracle checks read of DeviceInputs, with another case."""

    def __init__(self, inp, case):
        self.case, self.w, self.D, self.I = case, inp.w, inp.D, inp.I
        self.rank_begin = getattr(inp, "rank_begin", 0)


def _capture(step):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _poison(ts):
    for t in ts:
        t.fill_(float("nan"))


@pytest.mark.parametrize("name", ["gqa_fp8_binned", "mla_bf16_bimodal", "mla_bf16_longtail_sink"])
def test_decode_replays_with_changing_lengths(device, name):
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=CAP)
    inp = DeviceInputs(case, device).prepare(algo=dcp.DCP_ALGO_FAST)
    span = w.block_size * w.dcp_size
    seq_dev = inp.seq_lens          # [B] int32, read by the captured dcp_local_seq_lens

    def set_lengths(lens):
        seq_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        inp.block_table.copy_(torch.from_numpy(_table_for(case.block_table, lens, span)))

    def step():
        dcp.dcp_local_seq_lens(seq_dev, w.block_size, w.dcp_size, w.interleave, out=inp.local_lens)
        inp.step()

    set_lengths(DECODE_SETS[0])
    g = _capture(step)
    outs = [inp.po, inp.pl, inp.o, inp.lse]
    for rep, lens in enumerate(DECODE_SETS + DECODE_SETS[:2]):
        set_lengths(lens)
        _poison(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"{name}: replay {rep} lengths {lens}", flush=True)
        check_against_oracle(_View(inp, _truncated(case, lens)), outs)


@pytest.mark.parametrize("name", ["gqa_fp8_binned", "mla_bf16_bimodal"])
def test_verify_replays_with_changing_lengths(device, name):
    q_len = 2
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=CAP)
    inp = DeviceInputs(case, device)
    run = VerifyRun(inp, make_verify_queries(w, case.batch, q_len, device), algo=dcp.DCP_ALGO_FAST)
    span = w.block_size * w.dcp_size
    B = case.batch
    ql_dev = torch.empty(B * q_len, dtype=torch.int32, device=device)
    local_flat = run.local_lens.view(B * q_len, w.dcp_size)

    def set_lengths(lens):
        ql_dev.copy_(torch.from_numpy(verify_query_lens(lens, q_len).reshape(-1)))
        inp.block_table.copy_(torch.from_numpy(_table_for(case.block_table, lens, span)))

    def step():
        dcp.dcp_local_seq_lens(ql_dev, w.block_size, w.dcp_size, w.interleave, out=local_flat)
        run.step()

    set_lengths(VERIFY_SETS[0])
    g = _capture(step)
    outs = [run.po, run.pl, run.o, run.lse]
    Hq, Dv = w.num_q_heads, w.head_dim_v
    for rep, lens in enumerate(VERIFY_SETS + VERIFY_SETS[:1]):
        set_lengths(lens)
        _poison(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"{name} q_len {q_len}: replay {rep} lengths {lens}", flush=True)
        view = _View(inp, _truncated(case, lens))
        res = (run.po, run.pl, run.o.view(B, q_len, Hq, Dv), run.lse.view(B, q_len, Hq))
        check_verify_against_oracle(_VerifyView(run, view), res)


class _VerifyView:
    def __init__(self, run, view):
        self.inputs, self.q, self.q_len, self.rank_begin = view, run.q, run.q_len, run.rank_begin


@pytest.mark.parametrize("name,seg_rank", [("mla_bf16_longtail_sink", 0), ("gqa_fp8_binned", 7)])
def test_segment_replays_with_changing_lengths(device, name, seg_rank):
    window = 128
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=CAP)
    inp = DeviceInputs(case, device).prepare(algo=dcp.DCP_ALGO_FAST)
    seg = make_segment(w, case.seq_lens, window, case.k_scale, case.v_scale, device)
    sgi = SegmentInputs(inp, seg, device)
    span = w.block_size * w.dcp_size
    seq_dev = inp.seq_lens

    def set_lengths(lens):
        seq_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        inp.block_table.copy_(torch.from_numpy(_table_for(case.block_table, lens, span)))
        sgi.lens.copy_(torch.from_numpy(np.minimum(np.asarray(lens), window).astype(np.int32)))

    def step():
        dcp.dcp_local_seq_lens(seq_dev, w.block_size, w.dcp_size, w.interleave, out=inp.local_lens)
        inp.partial()
        sgi.fold(seg_rank, algo=dcp.DCP_ALGO_FAST)
        inp.merge()

    set_lengths(DECODE_SETS[0])
    g = _capture(step)
    outs = [inp.po, inp.pl, inp.o, inp.lse]
    for rep, lens in enumerate(DECODE_SETS):
        set_lengths(lens)
        _poison(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"{name} segment on rank {seg_rank}: replay {rep} lengths {lens}", flush=True)
        n = np.minimum(np.asarray(lens), window)
        seg_view = dataclasses.replace(seg, lens=n.astype(np.int32), k=[seg.k[b][:int(x)] for b, x in enumerate(n)],
                                       v=None if seg.v is None else [seg.v[b][:int(x)] for b, x in enumerate(n)])
        check_segment_against_oracle(_View(inp, _truncated(case, lens)), seg_view, seg_rank, outs)
