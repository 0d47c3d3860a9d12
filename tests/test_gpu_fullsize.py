"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (all ranks, MFMA kernels, the same seeded batch, pools
pre-filled with NaN bit patterns so that a read of an unwritten slot
poisons the result). Every request's merged output and LSE is compared with
the float64 oracle (full softmax over the unsharded sequence); every rank's
partial is compared with the oracle's partial over the tokens that rank owns
for a sample of requests (shortest, median, longest, one seeded pick).

Each workload runs once on the GPU; its requests are then checked in chunks
(one test per chunk), so that no single test holds the CPU oracle for long.
"""

import gc

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from tests.harness import check_against_oracle, check_segment_against_oracle, check_verify_against_oracle
from workloads import get_workload, make_case
from workloads.device import DeviceInputs

pytestmark = pytest.mark.gpu

_RUN = {}  # the one workload whose GPU result is held: name -> (inputs, extra, host result)


@pytest.fixture(scope="module", autouse=True)
def _release_at_end():
    yield
    _RUN.clear()
    gc.collect()
    torch.cuda.empty_cache()


def _hold(name, make):
    if name not in _RUN:
        _RUN.clear()
        gc.collect()
        torch.cuda.empty_cache()
        _RUN[name] = make()
    return _RUN[name]


def _sample(lens, seed):
    order = np.argsort(lens, kind="stable")
    picks = {int(order[0]), int(order[len(order) // 2]), int(order[-1])}
    picks.add(int(np.random.default_rng(seed).integers(0, len(lens))))
    return sorted(picks)


def _chunk(n, i, k):
    lo, hi = (n * i) // k, (n * (i + 1)) // k
    return list(range(lo, hi))


DECODE = [("gqa_fp8_binned", 8), ("mla_bf16_bimodal", 4), ("mla_bf16_longtail_sink", 4)]


@pytest.mark.parametrize("name,chunk,chunks", [(n, i, k) for n, k in DECODE for i in range(k)])
def test_full_size_every_request(device, name, chunk, chunks):
    def make():
        w = get_workload(name)
        case = make_case(w, device=device)
        inp = DeviceInputs(case, device, fill="nan")
        res = inp.run(algo=dcp.DCP_ALGO_AUTO)
        o, lse = res[2].float(), res[3]
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        host = tuple(t.float().cpu() for t in res)
        return inp, None, host
    inp, _, host = _hold(name, make)
    case = inp.case
    reqs = _chunk(case.batch, chunk, chunks)
    sampled = [b for b in _sample(case.seq_lens, case.workload.seed) if b in reqs]
    print(f"{name}: requests {reqs[0]}..{reqs[-1]} ({int(case.seq_lens[reqs].sum())} tokens), "
          f"partials of {sampled}", flush=True)
    check_against_oracle(inp, host, requests=[b for b in reqs if b not in sampled], check_parts=False)
    if sampled:
        check_against_oracle(inp, host, requests=sampled)


VERIFY = [("gqa_fp8_binned_q2", 8), ("gqa_bf16_32k_q4", 1), ("mla_bf16_bimodal_q2", 4)]


@pytest.mark.parametrize("name,chunk,chunks", [(n, i, k) for n, k in VERIFY for i in range(k)])
def test_verify_full_size_every_request(device, name, chunk, chunks):
    """Multi-token decode at the verification workloads' full sizes, in the
    launch configuration bench.py times."""
    from workloads import get_verify_workload, make_verify_queries
    from workloads.device import VerifyRun

    def make():
        vw = get_verify_workload(name)
        w = vw.geometry()
        case = make_case(w, device=device)
        inp = DeviceInputs(case, device, fill="nan")
        run = VerifyRun(inp, make_verify_queries(w, case.batch, vw.q_len, device), algo=dcp.DCP_ALGO_AUTO)
        res = run.run()
        assert torch.isfinite(res[2].float()).all() and torch.isfinite(res[3]).all()
        host = tuple(t.float().cpu() for t in res)
        run.q = run.q.cpu()
        return inp, run, host
    inp, run, host = _hold(name, make)
    case = inp.case
    reqs = _chunk(case.batch, chunk, chunks)
    sampled = [b for b in _sample(case.seq_lens, case.workload.seed + 1)[:3] if b in reqs]
    print(f"{name}: requests {reqs[0]}..{reqs[-1]}, partials of {sampled}", flush=True)
    check_verify_against_oracle(run, host, requests=[b for b in reqs if b not in sampled], check_parts=False)
    if sampled:
        check_verify_against_oracle(run, host, requests=sampled)


SEGMENT = [("mla_bf16_longtail_sink_swa128", 2), ("gqa_fp8_binned_swa128", 8)]


@pytest.mark.parametrize("name,chunk,chunks", [(n, i, k) for n, k in SEGMENT for i in range(k)])
def test_segment_full_size_every_request(device, name, chunk, chunks):
    """Decode with a replicated segment at full size, in bench.py's launch
    configuration."""
    from workloads import get_segment_workload, make_segment
    from workloads.device import SegmentInputs

    sw = get_segment_workload(name)

    def make():
        w = sw.geometry()
        case = make_case(w, device=device)
        inp = DeviceInputs(case, device, fill="nan")
        seg = make_segment(w, case.seq_lens, sw.window, case.k_scale, case.v_scale, device)
        sgi = SegmentInputs(inp, seg, device)
        inp.prepare(algo=dcp.DCP_ALGO_AUTO)
        inp.partial()
        sgi.fold(sw.seg_rank)
        inp.merge()
        torch.cuda.synchronize()
        res = (inp.po, inp.pl, inp.o, inp.lse)
        assert torch.isfinite(res[2].float()).all() and torch.isfinite(res[3]).all()
        host = tuple(t.float().cpu() for t in res)
        return inp, seg, host
    inp, seg, host = _hold(name, make)
    case = inp.case
    reqs = _chunk(case.batch, chunk, chunks)
    sampled = [b for b in _sample(case.seq_lens, case.workload.seed + 2)[:2] if b in reqs]
    print(f"{name}: requests {reqs[0]}..{reqs[-1]}, partials of {sampled}", flush=True)
    check_segment_against_oracle(inp, seg, sw.seg_rank, host, requests=[b for b in reqs if b not in sampled],
                                 check_parts=False)
    if sampled:
        check_segment_against_oracle(inp, seg, sw.seg_rank, host, requests=sampled)
