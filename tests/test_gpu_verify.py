"""GPU parity of multi-token decode (speculative verification), through the
C ABI (dcp_partial_verify_attn, then dcp_lse_merge over batch * q_len rows),
against the float64 oracle (oracle.attention.verify_attention and its
per-rank partials). Tolerances as for decode (tests/harness.TOL).

Lengths include requests made only of new tokens (q_len = L: the first query
sees one position, so most ranks see nothing for it while later queries see
tokens there), ragged tiles, and q_len values that fill the GQA kernel's 16
score columns exactly, in part, and over several units.
"""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from workloads import get_workload, make_case
from workloads.generate import make_verify_queries
from tests.harness import DeviceInputs, VerifyRun, check_verify_against_oracle

pytestmark = pytest.mark.gpu

GEN, FAST = dcp.DCP_ALGO_GENERIC, dcp.DCP_ALGO_FAST

# name: (lengths, each >= the largest q_len, q_len values)
VERIFY = {
    "gqa_fp32_tiny": ([8, 37, 100], [1, 3, 8]),
    "gqa_bf16_32k": ([8, 9, 16, 17, 33, 100, 257, 1000, 4099], [1, 2, 3, 4, 5, 8]),
    "gqa_fp8_binned": ([8, 9, 63, 64, 65, 511, 513, 3000, 10000], [1, 2, 3, 8]),
    "mla_bf16_bimodal": ([8, 31, 33, 65, 700, 2000, 4097], [1, 2, 4]),
    "mla_bf16_longtail_sink": ([8, 37, 600, 2049], [2, 3]),
}


def _algos(name):
    return [GEN] if name == "gqa_fp32_tiny" else [GEN, FAST]


@pytest.mark.parametrize("name", sorted(VERIFY))
def test_verify_small(device, name):
    w = get_workload(name)
    lens, q_lens = VERIFY[name]
    case = make_case(w, device=device, seq_lens=lens)
    inp = DeviceInputs(case, device)
    for q_len in q_lens:
        q = make_verify_queries(w, case.batch, q_len, device)
        for algo in _algos(name):
            run = VerifyRun(inp, q, algo=algo)
            check_verify_against_oracle(run, run.run())


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_bimodal"])
def test_one_query_token_is_decode(device, name):
    """q_len = 1 runs the decode kernels: results equal dcp_partial_decode_attn's bit for bit."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[5, 300, 2000])
    inp = DeviceInputs(case, device)
    po_d, pl_d, _, _ = [t.clone() for t in inp.run(algo=FAST)]
    run = VerifyRun(inp, case.q.to(device)[:, None].contiguous(), algo=FAST)
    po, pl, _, _ = run.run()
    assert torch.equal(po[:, :, 0], po_d) and torch.equal(pl[:, :, 0], pl_d)


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_longtail_sink"])
def test_verify_rank_subsets(device, name):
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[70, 4, 300, 2000])
    inp = DeviceInputs(case, device)
    q = make_verify_queries(w, case.batch, 4, device)
    for rb, rc in [(0, 1), (1, 2), (inp.D - 1, 1)]:
        run = VerifyRun(inp, q, algo=FAST, rank_begin=rb, rank_count=rc)
        check_verify_against_oracle(run, run.run())


def test_verify_rejects_bad_q_len(device):
    w = get_workload("gqa_bf16_32k")
    case = make_case(w, device=device, seq_lens=[40])
    inp = DeviceInputs(case, device)
    kv = inp.cache.descriptor()
    for q_len in (0, 65):
        with pytest.raises(dcp.DcpError):
            dcp.dcp_partial_verify_attn_workspace_size(1, q_len, w.num_q_heads, dcp.DCP_BF16, kv, inp.D)


def test_verify_matches_across_kernels(device):
    """The MFMA path with several units per request (q_len = 8 > 16 / group)
    against the generic kernel on a longer batch."""
    w = get_workload("gqa_fp8_binned")
    case = make_case(w, device=device, seq_lens=[20000, 8, 700])
    inp = DeviceInputs(case, device)
    q = make_verify_queries(w, case.batch, 8, device)
    a = [t.clone() for t in VerifyRun(inp, q, algo=FAST).run()]
    b = VerifyRun(inp, q, algo=GEN).run()
    np.testing.assert_allclose(a[2].float().cpu().numpy(), b[2].float().cpu().numpy(), atol=2e-2)
    fin = torch.isfinite(b[1])
    assert torch.equal(torch.isfinite(a[1]), fin)
    assert (a[1][fin] - b[1][fin]).abs().max().item() <= 1e-3


def test_verify_many_pairs_per_thread_chunk(device):
    """More (rank, request) pairs than the attention kernel's threads (200
    requests x 8 ranks > 256), so each thread of its split search sums a chunk
    of several pairs, with two token groups per pair (q_len = 3 > 16 / group)
    and 8 KV heads: a worker's first unit is found by KV head and token group
    inside its pair. Short ragged lengths keep the oracle cheap; every request
    is checked."""
    w = get_workload("gqa_fp8_binned")
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(3, 400, size=200)]
    case = make_case(w, device=device, seq_lens=lens)
    inp = DeviceInputs(case, device)
    q = make_verify_queries(w, case.batch, 3, device)
    for algo in (FAST, GEN):
        run = VerifyRun(inp, q, algo=algo)
        check_verify_against_oracle(run, run.run())
