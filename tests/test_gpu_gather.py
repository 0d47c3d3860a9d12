"""GPU parity of the chunked-prefill context gather (dcp_gather_context)
through the C ABI: bit for bit against the oracle's gather over the same
stored pools (copied to the host), for MLA latent rows and GQA K/V rows in a
row layout, every stored format, contexts shorter than the cached sequences,
empty requests and unmapped virtual blocks (zero rows); at full size, every
gathered row against the canonical rows the pools were filled from.
"""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from oracle import gather as ogather
from workloads import get_workload, make_case
from workloads.generate import stored_numpy
from tests.harness import DeviceInputs

pytestmark = pytest.mark.gpu

RAW = {1: torch.uint8, 2: torch.int16, 4: torch.int32}


def _bits(t):
    return t.view(RAW[t.element_size()]).cpu().numpy()


def _gather(inp, ctx_lens, with_v, table=None):
    w, dev = inp.w, inp.q.device
    cu = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(np.int64)
    T = int(cu[-1])
    dt = inp.cache.dtype
    out_k = torch.full((T, w.num_kv_heads, w.head_dim_k), 0, dtype=dt, device=dev)
    out_k.view(torch.uint8).fill_(0xA5)
    out_v = None
    if with_v:
        out_v = torch.empty((T, w.num_kv_heads, w.head_dim_v), dtype=dt, device=dev)
        out_v.view(torch.uint8).fill_(0xA5)
    bt = inp.block_table if table is None else torch.from_numpy(table).to(dev)
    dcp.dcp_gather_context(inp.cache.descriptor(0), inp.D, inp.I, bt, torch.from_numpy(cu).to(dev), T, out_k, out_v)
    torch.cuda.synchronize()
    return out_k, out_v


def _oracle(inp, ctx_lens, with_v, table=None):
    kp = _bits(inp.cache.k)
    vp = None
    if with_v:
        vp = np.swapaxes(_bits(inp.cache.v), 3, 4)        # token-major pool -> the oracle's [.., dim, token] view
    t = inp.block_table_np if table is None else table
    return ogather.gather_context(kp, vp, t, ctx_lens, inp.bs, inp.D, inp.I)


CASES = [
    # (workload, v_layout, with_v, sequence lengths)
    ("mla_bf16_bimodal", "dim_major", False, [1, 31, 64, 65, 700, 0, 2000]),
    ("mla_bf16_longtail_sink", "dim_major", False, [5, 600, 2049]),
    ("gqa_bf16_32k", "token_major", True, [1, 15, 16, 17, 100, 0, 1000]),
    ("gqa_fp8_binned", "token_major", True, [1, 63, 64, 65, 513, 3000]),
    ("gqa_fp8_binned", "dim_major", False, [70, 5]),
    ("gqa_fp32_tiny", "token_major", True, [37, 100]),
]


@pytest.mark.parametrize("name,v_layout,with_v,lens", CASES)
def test_gather_bitexact(device, name, v_layout, with_v, lens):
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=lens)
    inp = DeviceInputs(case, device, v_layout=v_layout)
    rng = np.random.default_rng(len(lens))
    for ctx in (np.asarray(lens), np.maximum(np.asarray(lens) - rng.integers(0, 40, len(lens)), 0)):
        gk, gv = _gather(inp, ctx, with_v)
        ok, ov = _oracle(inp, ctx, with_v)
        assert np.array_equal(_bits(gk), ok.view(_bits(gk).dtype))
        if with_v:
            assert np.array_equal(_bits(gv), ov.view(_bits(gv).dtype))


def test_gather_unmapped_blocks_are_zero(device):
    w = get_workload("mla_bf16_bimodal")
    case = make_case(w, device=device, seq_lens=[2000, 1500])
    inp = DeviceInputs(case, device)
    table = inp.block_table_np.copy()
    table[0, 1] = -1                                       # a hole in request 0
    ctx = np.array([2000, 1500])
    gk, _ = _gather(inp, ctx, False, table)
    ok, _ = _oracle(inp, ctx, False, table)
    assert np.array_equal(_bits(gk), ok.view(np.int16))
    span = w.block_size * w.dcp_size
    assert np.all(_bits(gk)[span:2 * span] == 0)


def test_gather_errors(device):
    w = get_workload("gqa_fp8_binned")
    case = make_case(w, device=device, seq_lens=[100])
    inp = DeviceInputs(case, device)                       # V transposed inside a block: no row gather
    with pytest.raises(dcp.DcpError):
        _gather(inp, np.array([100]), True)
    wm = get_workload("mla_bf16_bimodal")
    cm = make_case(wm, device=device, seq_lens=[100])
    im = DeviceInputs(cm, device)
    out = torch.empty((100, 1, 576), dtype=torch.bfloat16, device=device)
    cu = torch.tensor([0, 100], dtype=torch.int64, device=device)
    with pytest.raises(dcp.DcpError):                      # MLA: the value is in the latent row
        dcp.dcp_gather_context(im.cache.descriptor(0), im.D, im.I, im.block_table, cu, 100, out, out)


def test_gather_full_size(device):
    """The whole context of the mla_bf16_bimodal batch (5.7M tokens), as bench.py
    gathers it; every row against the canonical rows the pools were filled from."""
    w = get_workload("mla_bf16_bimodal")
    case = make_case(w, device=device)
    inp = DeviceInputs(case, device, fill="zero")
    gk, _ = _gather(inp, case.seq_lens.astype(np.int64), False)
    cu = np.concatenate([[0], np.cumsum(case.seq_lens.astype(np.int64))])
    raw = gk.view(torch.int16)
    for b in range(case.batch):
        assert torch.equal(raw[cu[b]:cu[b + 1]], case.k[b].view(torch.int16)), f"request {b}"
