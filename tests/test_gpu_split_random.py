"""Randomised GPU parity of the stream-K split behind the MFMA kernels: the
GQA kernel's own split search, the MLA planner, the combine's cut records and
its pass over token groups without local tokens. Seeded random batches
(1 to 150 requests; long, short or partly empty lengths, so that units are
cut into one to many pieces and many ranks hold nothing), every rank or a
rank subset, decode and multi-token decode, through the C ABI; every rank's
partial and the merged rows are checked against the float64 oracle
(tests/harness.TOL) for every request.
"""

import numpy as np
import pytest

import sequence_sharded_paged_amd as dcp
from workloads import get_workload, make_case
from workloads.generate import make_verify_queries
from tests.harness import DeviceInputs, VerifyRun, check_against_oracle, check_verify_against_oracle

pytestmark = pytest.mark.gpu

FAST = dcp.DCP_ALGO_FAST


def _lengths(rng, kind, batch, cap):
    if kind == 0:  # long and ragged
        lens = rng.integers(0, cap, batch)
    elif kind == 1:  # short: most ranks empty
        lens = rng.integers(0, 200, batch)
    else:  # a third of the requests empty, the rest anywhere up to the cap
        lens = np.where(rng.random(batch) < 0.3, 0, rng.integers(1, cap, batch))
    return [int(x) for x in lens]


@pytest.mark.parametrize("name,cap", [("gqa_bf16_32k", 6000), ("gqa_fp8_binned", 6000),
                                      ("mla_bf16_bimodal", 2500)])
@pytest.mark.parametrize("seed", range(4))
def test_random_decode_batches(device, name, cap, seed):
    rng = np.random.default_rng(7000 + 13 * seed + len(name))
    batch = int(rng.choice([1, 3, 17, 64, 150] if name.startswith("gqa") else [1, 5, 23, 64]))
    lens = _lengths(rng, seed % 3, batch, cap)
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=lens)
    inp = DeviceInputs(case, device)
    D = inp.D
    rb, rc = (0, None) if seed % 2 == 0 else (int(rng.integers(0, D)), None)
    if rc is None and rb > 0:
        rc = int(rng.integers(1, D - rb + 1))
    print(f"{name} seed {seed}: {batch} requests, ranks {rb}+{rc or D - rb}", flush=True)
    res = inp.run(algo=FAST, rank_begin=rb, rank_count=rc)
    check_against_oracle(inp, res, rank_begin=rb)


@pytest.mark.parametrize("name,q_len", [("gqa_fp8_binned", 3), ("gqa_bf16_32k", 4), ("mla_bf16_bimodal", 2)])
def test_random_verify_batches(device, name, q_len):
    rng = np.random.default_rng(9100 + q_len)
    batch = 40 if name.startswith("gqa") else 12
    lens = [max(q_len, x) for x in _lengths(rng, 2, batch, 3000)]
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=lens)
    inp = DeviceInputs(case, device)
    q = make_verify_queries(w, case.batch, q_len, device)
    print(f"{name} verify q_len {q_len}: {batch} requests", flush=True)
    run = VerifyRun(inp, q, algo=FAST)
    check_verify_against_oracle(run, run.run())
