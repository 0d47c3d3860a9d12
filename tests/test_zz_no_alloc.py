"""dcp_partial_decode_attn_noalloc (the library's fixed device scratch as the
workspace) against dcp_partial_decode_attn with a caller-allocated workspace:
the same kernels on the same inputs, so every partial output and LSE must
agree bit for bit (NaN-filled outputs first, so an unwritten entry fails).

The no-allocation calls run back to back on one device and share its
scratch: for each workload a larger batch, then a smaller one (fewer
requests, tokens and split units than the plan the scratch still holds), then
an all-empty batch. Covers the GQA bf16 and fp8 kernels, both MLA workloads
and the generic kernel (which takes no workspace).
"""

import pytest
import torch

import sequence_sharded_paged_amd as dcp
from workloads import get_workload, make_case
from workloads.device import DeviceInputs

pytestmark = pytest.mark.gpu

CASES = [
    ("gqa_bf16_32k", dcp.DCP_ALGO_FAST, [[5000, 33, 0, 1200, 64, 9000, 17], [700, 1], [0, 0, 0]]),
    ("gqa_fp8_binned", dcp.DCP_ALGO_FAST, [[3000, 129, 7000, 1, 0, 20000, 513], [65, 2], [0, 0]]),
    ("mla_bf16_bimodal", dcp.DCP_ALGO_FAST, [[3000, 650, 9000, 1, 0, 4097, 31], [129, 2], [0]]),
    ("mla_bf16_longtail_sink", dcp.DCP_ALGO_FAST, [[40000, 5, 1500], [37], [0, 0]]),
    ("gqa_fp32_tiny", dcp.DCP_ALGO_AUTO, [[100, 37], [5], [0]]),
]


def _bits(t):
    return t.contiguous().view(torch.int32)


@pytest.mark.parametrize("name,algo,batches", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry(device, name, algo, batches):
    w = get_workload(name)
    runs = []
    for lens in batches:  # reference results first, with a workspace of the caller's
        inp = DeviceInputs(make_case(w, device=device, seq_lens=lens), device).prepare(algo=algo)
        inp.partial()
        torch.cuda.synchronize()
        runs.append((lens, inp, inp.po.clone(), inp.pl.clone()))
    for i, (lens, inp, ref_o, ref_l) in enumerate(runs):  # then the no-allocation calls, back to back
        print(f"{name}: no-allocation call {i}, lengths {lens}", flush=True)
        inp.po.fill_(float("nan"))
        inp.pl.fill_(float("nan"))
        dcp.dcp_partial_decode_attn_noalloc(inp.q, inp.kv, inp.block_table, inp.local_lens, inp.D, inp.rank_begin,
                                            inp.rank_count, w.softmax_scale, inp.po, inp.pl, algo=algo)
        torch.cuda.synchronize()
        assert torch.equal(_bits(inp.po), _bits(ref_o)), f"{name} call {i}: partial outputs differ"
        assert torch.equal(_bits(inp.pl), _bits(ref_l)), f"{name} call {i}: partial LSEs differ"


def test_noalloc_refuses_oversized_problem(device):
    """A problem whose workspace exceeds the fixed scratch is refused with
    DCP_ERR_SCRATCH on the host and launches nothing: the output buffer keeps
    its contents. (The call reads no buffer before refusing, so small
    stand-ins are passed for the 2^20-request operands.)"""
    import ctypes
    w = get_workload("mla_bf16_bimodal")
    inp = DeviceInputs(make_case(w, device=device, seq_lens=[64, 3]), device).prepare(algo=dcp.DCP_ALGO_FAST)
    big_b = 1 << 20  # 2^23 split units over 8 ranks
    need = dcp.dcp_partial_decode_attn_workspace_size(big_b, w.num_q_heads, dcp.DCP_BF16, inp.kv, inp.rank_count,
                                                      dcp.DCP_ALGO_FAST)
    assert need > dcp.DCP_NOALLOC_SCRATCH_BYTES
    buf = torch.full((64,), 7.0, device=device)
    p = ctypes.c_void_p(buf.data_ptr())
    st = dcp.native.lib().dcp_partial_decode_attn_noalloc(
        p, dcp.DCP_BF16, big_b, w.num_q_heads, ctypes.byref(inp.kv), p, 1, 1, p, inp.D, 0, inp.rank_count,
        ctypes.c_float(w.softmax_scale), dcp.DCP_ALGO_FAST, p, p, dcp.native._stream())
    assert st == dcp.DCP_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(buf == 7.0)
