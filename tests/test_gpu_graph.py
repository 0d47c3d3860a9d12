"""The hot path under HIP graph capture: a decode step (every rank's partials
and the merge), a multi-token verification step, a decode step with a
replicated segment, a chunked-prefill KV write, the context gather and the
block-table check are captured once and replayed several times, with eager work (the outputs
overwritten) between replays; every replay must reproduce the eager result bit
for bit (the kernels are deterministic and launch only kernels: no
allocation, copy, memset or synchronisation inside a call)."""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from tests.harness import DeviceInputs, SegmentInputs, VerifyRun
from workloads import get_kv_write_workload, get_workload, make_case, make_kv_write_case, make_verify_queries
from workloads.generate import TORCH_FORMAT, make_segment

pytestmark = pytest.mark.gpu


def _capture(step):
    """Warm up on a side stream (as torch asks), then capture one call of step."""
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


def _reset(outs):
    """The same sentinel before the eager call and before every replay, so
    that elements a call does not write compare equal too."""
    for t in outs:
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(85)


def _replay_matches(g, outs, refs, reps=3):
    for rep in range(reps):
        _reset(outs)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, refs)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"


@pytest.mark.parametrize("name,lens", [("gqa_fp8_binned", [3000, 129, 7000, 1]),
                                       ("gqa_bf16_32k", [900, 2100, 5]),
                                       ("mla_bf16_bimodal", [3000, 650, 9000]),
                                       ("mla_bf16_longtail_sink", [4000, 33])])
def test_decode_step_replays(device, name, lens):
    w = get_workload(name)
    inp = DeviceInputs(make_case(w, device=device, seq_lens=lens), device).prepare(algo=dcp.DCP_ALGO_FAST)
    outs = [inp.po, inp.pl, inp.o, inp.lse]
    _reset(outs)
    inp.step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    g = _capture(inp.step)
    _replay_matches(g, outs, refs)


def test_verify_step_replays(device):
    w = get_workload("gqa_fp8_binned")
    case = make_case(w, device=device, seq_lens=[2500, 40, 6100])
    inp = DeviceInputs(case, device)
    run = VerifyRun(inp, make_verify_queries(w, case.batch, 2, device), algo=dcp.DCP_ALGO_FAST)
    outs = [run.po, run.pl, run.o, run.lse]
    _reset(outs)
    run.run()
    refs = [t.clone() for t in outs]
    g = _capture(run.step)
    _replay_matches(g, outs, refs)


def test_kv_write_replays(device):
    w = get_kv_write_workload("kvw_gqa_fp8_chunk")
    g = w.geometry()
    case = make_kv_write_case(w, device)
    R, N, H, bs = g.dcp_size, case.num_blocks, g.num_kv_heads, g.block_size
    pool = dcp.PagedKVCache(R, N, bs, H, g.head_dim_k, g.head_dim_v, TORCH_FORMAT[g.kv_format], mla=g.mla,
                            device=device, k_scale=case.k_scale, v_scale=case.v_scale)
    desc = pool.descriptor()
    positions = torch.from_numpy(case.positions).to(device)
    reqs = torch.from_numpy(case.req_indices).to(device)
    table = torch.from_numpy(case.block_table).to(device)
    slots = torch.empty((R, w.tokens), dtype=torch.int64, device=device)

    def step():
        dcp.dcp_slot_mapping(positions, reqs, table, bs, R, g.interleave, out=slots)
        dcp.dcp_kv_cache_write(case.k_new, case.v_new, slots, desc)

    outs = [slots, pool.k.view(torch.uint8), pool.v.view(torch.uint8)]
    _reset(outs)
    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    gr = _capture(step)
    _replay_matches(gr, outs, refs)


@pytest.mark.parametrize("name,seg_rank", [("mla_bf16_longtail_sink", 0), ("gqa_fp8_binned", 7)])
def test_segment_step_replays(device, name, seg_rank):
    """Partials, the replicated segment folded into one rank, then the merge."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[1500, 90, 4000])
    inp = DeviceInputs(case, device).prepare(algo=dcp.DCP_ALGO_FAST)
    seg = SegmentInputs(inp, make_segment(w, case.seq_lens, 128, case.k_scale, case.v_scale, device), device)

    def step():
        inp.partial()
        seg.fold(seg_rank, algo=dcp.DCP_ALGO_FAST)
        inp.merge()

    outs = [inp.po, inp.pl, inp.o, inp.lse]
    _reset(outs)
    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    g = _capture(step)
    _replay_matches(g, outs, refs)


@pytest.mark.parametrize("name,v_layout,with_v", [("mla_bf16_bimodal", "dim_major", False),
                                                  ("gqa_fp8_binned", "token_major", True)])
def test_gather_replays(device, name, v_layout, with_v):
    w = get_workload(name)
    lens = [3000, 77, 5200]
    inp = DeviceInputs(make_case(w, device=device, seq_lens=lens), device, v_layout=v_layout)
    ctx = np.array([2999, 77, 4100])
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)).to(device)
    T = int(ctx.sum())
    out_k = torch.empty((T, w.num_kv_heads, w.head_dim_k), dtype=inp.cache.dtype, device=device)
    out_v = torch.empty((T, w.num_kv_heads, w.head_dim_v), dtype=inp.cache.dtype, device=device) if with_v else None
    desc = inp.cache.descriptor(0)

    def step():
        dcp.dcp_gather_context(desc, inp.D, inp.I, inp.block_table, cu, T, out_k, out_v)

    outs = [out_k.view(torch.uint8)] + ([out_v.view(torch.uint8)] if with_v else [])
    _reset(outs)
    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    g = _capture(step)
    _replay_matches(g, outs, refs)


def test_block_table_check_replays(device):
    """The check clears its counter with a kernel, so a replay counts afresh."""
    w = get_workload("gqa_fp8_binned")
    case = make_case(w, device=device, seq_lens=[3000, 70, 9000])
    inp = DeviceInputs(case, device)
    table = inp.block_table.clone()
    table[0, 0] = inp.cache.num_blocks + 5  # one entry past the pool
    table[2, 1] = -3                         # one missing entry
    seq_lens = inp.seq_lens
    cnt = torch.empty(1, dtype=torch.int32, device=device)

    def step():
        dcp.dcp_check_block_table(table, seq_lens, w.block_size, w.dcp_size, inp.cache.num_blocks, out=cnt)

    _reset([cnt])
    step()
    torch.cuda.synchronize()
    assert int(cnt.item()) == 2
    refs = [cnt.clone()]
    g = _capture(step)
    _replay_matches(g, [cnt], refs)
