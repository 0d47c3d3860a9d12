"""GPU parity of the replicated segment (a sliding-window cache kept whole on
every rank, counted by one): dcp_partial_decode_attn, then
dcp_partial_segment_attn folding each request's segment into rank seg_rank's
partial, then dcp_lse_merge with the sink, all through the C ABI, against the
float64 oracle (attention over the sequence and the segment together; the
per-rank partials with the segment on the designated rank only).
"""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from workloads import get_workload, make_case
from workloads.generate import make_segment
from tests.harness import DeviceInputs, SegmentInputs, check_segment_against_oracle

pytestmark = pytest.mark.gpu

GEN, FAST, AUTO = dcp.DCP_ALGO_GENERIC, dcp.DCP_ALGO_FAST, dcp.DCP_ALGO_AUTO

# Windows from one token to several hundred (300, 400, 600: a segment pool of
# many blocks, units cut between workers in the MFMA path).
CASES = {
    # name: (lengths, windows)
    "gqa_fp32_tiny": ([8, 37, 100], [1, 40]),
    "gqa_bf16_32k": ([1, 17, 100, 257, 1000, 0], [1, 128, 300]),
    "gqa_fp8_binned": ([1, 64, 65, 513, 3000, 0], [64, 128, 400]),
    "mla_bf16_bimodal": ([1, 33, 65, 700, 2000], [32, 128, 600]),
    "mla_bf16_longtail_sink": ([5, 37, 600, 2049], [128]),
}


def _algos(name):
    # fp32 KV has no MFMA kernel: FAST refuses it, AUTO takes the generic kernel
    return [GEN, AUTO] if name == "gqa_fp32_tiny" else [GEN, FAST]


def _run(inp, sgi, seg_rank, algo):
    inp.prepare(algo=algo)
    inp.partial()
    sgi.fold(seg_rank, algo=algo)
    inp.merge()
    torch.cuda.synchronize()
    return inp.po, inp.pl, inp.o, inp.lse


@pytest.mark.parametrize("name", sorted(CASES))
def test_segment_small(device, name):
    w = get_workload(name)
    lens, windows = CASES[name]
    case = make_case(w, device=device, seq_lens=lens)
    inp = DeviceInputs(case, device)
    for window in windows:
        seg = make_segment(w, case.seq_lens, window, case.k_scale, case.v_scale, device)
        sgi = SegmentInputs(inp, seg, device)
        for seg_rank in (0, inp.D - 1):
            for algo in _algos(name):
                res = _run(inp, sgi, seg_rank, algo)
                check_segment_against_oracle(inp, seg, seg_rank, res)


def test_other_ranks_and_empty_segment_unchanged(device):
    """A segment counted by a rank outside the computed ones, or an empty
    segment, leaves every partial bit for bit as dcp_partial_decode_attn wrote it."""
    w = get_workload("gqa_fp8_binned")
    case = make_case(w, device=device, seq_lens=[300, 70, 2000])
    inp = DeviceInputs(case, device)
    seg = make_segment(w, case.seq_lens, 128, case.k_scale, case.v_scale, device)
    sgi = SegmentInputs(inp, seg, device)
    inp.prepare(algo=FAST, rank_begin=2, rank_count=3)
    inp.partial()
    ref_o, ref_l = inp.po.clone(), inp.pl.clone()
    sgi.fold(0, algo=FAST)                      # rank 0 is not among ranks 2..4: nothing launched
    sgi.fold(7, algo=FAST)
    torch.cuda.synchronize()
    assert torch.equal(inp.po, ref_o) and torch.equal(inp.pl, ref_l)
    empty = make_segment(w, case.seq_lens, 0, case.k_scale, case.v_scale, device)
    sge = SegmentInputs(inp, empty, device)
    sge.fold(3, algo=FAST)
    torch.cuda.synchronize()
    assert torch.equal(inp.po, ref_o) and torch.equal(inp.pl, ref_l)


def test_segment_on_a_rank_with_no_tokens(device):
    """Requests shorter than one rank's share: the designated rank's partial is the segment's alone."""
    w = get_workload("mla_bf16_bimodal")
    case = make_case(w, device=device, seq_lens=[3, 1, 7])
    inp = DeviceInputs(case, device)
    seg = make_segment(w, case.seq_lens + 50, 40, case.k_scale, case.v_scale, device)
    sgi = SegmentInputs(inp, seg, device)
    res = _run(inp, sgi, inp.D - 1, FAST)
    check_segment_against_oracle(inp, seg, inp.D - 1, res)
    assert torch.isfinite(res[1][inp.D - 1]).all()
