"""The hot path under HIP graph capture: a decode step (every rank's partials
and the merge), a multi-token verification step and a chunked-prefill KV write
are captured once and replayed several times, with eager work (the outputs
overwritten) between replays; every replay must reproduce the eager result bit
for bit (the kernels are deterministic and launch only kernels: no
allocation, copy, memset or synchronisation inside a call)."""

import pytest
import torch

import sequence_sharded_paged_amd as dcp
from tests.harness import DeviceInputs, VerifyRun
from workloads import get_kv_write_workload, get_workload, make_case, make_kv_write_case, make_verify_queries
from workloads.generate import TORCH_FORMAT

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
