"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (all ranks, MFMA kernels, the same seeded batch). The oracle
recomputes a sample of requests one by one (shortest, median, longest, and
one seeded pick): merged output against full softmax over the unsharded
sequence, and every rank's partial against the oracle's partial over the
tokens that rank owns."""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from tests.harness import DeviceInputs, check_against_oracle
from workloads import get_workload, make_case

pytestmark = pytest.mark.gpu


def _sample(lens, seed):
    order = np.argsort(lens, kind="stable")
    picks = {int(order[0]), int(order[len(order) // 2]), int(order[-1])}
    picks.add(int(np.random.default_rng(seed).integers(0, len(lens))))
    return sorted(picks)


@pytest.mark.parametrize("name,max_requests", [("gqa_fp8_binned", 4), ("mla_bf16_bimodal", 4),
                                               ("mla_bf16_longtail_sink", 2)])
def test_full_size_sampled(device, name, max_requests):
    w = get_workload(name)
    case = make_case(w, device=device)
    inp = DeviceInputs(case, device, fill="zero")
    res = inp.run(algo=dcp.DCP_ALGO_AUTO)
    # properties at full size for every request: finite outputs, LSE defined
    o, lse = res[2].float(), res[3]
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    reqs = _sample(case.seq_lens, w.seed)[:max_requests] if max_requests < 4 else _sample(case.seq_lens, w.seed)
    if name == "mla_bf16_longtail_sink":
        order = np.argsort(case.seq_lens)
        reqs = [int(order[0]), int(order[-1])]
    print(f"{name}: checking requests {reqs} of lengths {[int(case.seq_lens[b]) for b in reqs]}", flush=True)
    check_against_oracle(inp, res, requests=reqs)


@pytest.mark.parametrize("name", ["gqa_fp8_binned_q2", "gqa_bf16_32k_q4", "mla_bf16_bimodal_q2"])
def test_verify_full_size_sampled(device, name):
    """Multi-token decode at the verification workloads' full sizes, in the
    launch configuration bench.py times; sampled requests against the oracle."""
    from tests.harness import VerifyRun, check_verify_against_oracle
    from workloads import get_verify_workload, make_verify_queries
    vw = get_verify_workload(name)
    w = vw.geometry()
    case = make_case(w, device=device)
    inp = DeviceInputs(case, device, fill="zero")
    run = VerifyRun(inp, make_verify_queries(w, case.batch, vw.q_len, device), algo=dcp.DCP_ALGO_AUTO)
    res = run.run()
    assert torch.isfinite(res[2].float()).all() and torch.isfinite(res[3]).all()
    reqs = _sample(case.seq_lens, w.seed + 1)[:3]
    print(f"{name}: checking requests {reqs} of lengths {[int(case.seq_lens[b]) for b in reqs]}", flush=True)
    check_verify_against_oracle(run, res, requests=reqs)


@pytest.mark.parametrize("name", ["mla_bf16_longtail_sink_swa128", "gqa_fp8_binned_swa128"])
def test_segment_full_size_sampled(device, name):
    """Decode with a replicated segment at full size, in bench.py's launch
    configuration; sampled requests against the oracle."""
    from tests.harness import SegmentInputs, check_segment_against_oracle
    from workloads import get_segment_workload, make_segment
    sw = get_segment_workload(name)
    w = sw.geometry()
    case = make_case(w, device=device)
    inp = DeviceInputs(case, device, fill="zero")
    seg = make_segment(w, case.seq_lens, sw.window, case.k_scale, case.v_scale, device)
    sgi = SegmentInputs(inp, seg, device)
    inp.prepare(algo=dcp.DCP_ALGO_AUTO)
    inp.partial()
    sgi.fold(sw.seg_rank)
    inp.merge()
    torch.cuda.synchronize()
    res = (inp.po, inp.pl, inp.o, inp.lse)
    assert torch.isfinite(res[2].float()).all() and torch.isfinite(res[3]).all()
    reqs = _sample(case.seq_lens, w.seed + 2)[:2]
    print(f"{name}: checking requests {reqs} of lengths {[int(case.seq_lens[b]) for b in reqs]}", flush=True)
    check_segment_against_oracle(inp, seg, sw.seg_rank, res, requests=reqs)
