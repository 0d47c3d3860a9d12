"""GPU parity: every HIP kernel against the CPU oracle, through the C ABI.

Integer work (local lengths, slot mapping) must be bit-exact; attention must
meet the tolerances in harness.TOL on both the per-rank partials and the
merged result. Pools are pre-filled with NaN bit patterns so that any read of
a slot the layout did not fill poisons the output.
"""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from oracle import attention as oatt
from oracle import formats as ofmt
from oracle import layout as olay
from workloads import get_workload, make_case
from tests.harness import DeviceInputs, check_against_oracle, check_lse, check_rows, TOL

pytestmark = pytest.mark.gpu

GEN, FAST = dcp.DCP_ALGO_GENERIC, dcp.DCP_ALGO_FAST


# ---------------------------------------------------------------------------
# slot mapping and local lengths (bit-exact)
# ---------------------------------------------------------------------------
LAYOUTS = [(bs, D, I) for bs in (1, 2, 16, 64) for D in (1, 2, 3, 4, 8) for I in (1, 2, 16, 64) if bs % I == 0]


@pytest.mark.parametrize("bs,D,I", LAYOUTS)
def test_local_seq_lens_bitexact(device, bs, D, I):
    rng = np.random.default_rng(bs * 1000 + D * 10 + I)
    lens = np.concatenate([[0, 1, 2, bs * D - 1, bs * D, bs * D + 1, 1 << 20, (1 << 20) + 37],
                           rng.integers(0, 300000, size=40)]).astype(np.int32)
    got = dcp.dcp_local_seq_lens(torch.from_numpy(lens).to(device), bs, D, I).cpu().numpy()
    ref = olay.local_seq_lens(lens, bs, D, I)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("bs,D,I", LAYOUTS)
def test_slot_mapping_bitexact(device, bs, D, I):
    rng = np.random.default_rng(bs * 7 + D * 3 + I)
    span = bs * D
    lens = [1, span - 1, 3 * span + 5, 600]
    nvb = [(L + span - 1) // span for L in lens]
    width = max(nvb) + 2
    table = np.full((len(lens), width), -1, dtype=np.int32)
    perm = rng.permutation(sum(nvb) + 5).astype(np.int32)
    pos = 0
    for b, n in enumerate(nvb):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    table[3, 1] = -1                                           # a hole: unallocated block
    positions = np.concatenate([np.arange(L) for L in lens] + [[-1, -5, width * span, width * span + 3, 7, 0]])
    reqs = np.concatenate([np.full(L, b) for b, L in enumerate(lens)] + [[0, 1, 2, 3, 9, -1]])
    got = dcp.dcp_slot_mapping(torch.from_numpy(positions.astype(np.int64)).to(device),
                               torch.from_numpy(reqs.astype(np.int32)).to(device),
                               torch.from_numpy(table).to(device), bs, D, I).cpu().numpy()
    ref = olay.slot_mapping(positions, reqs, table, bs, D, I)
    assert np.array_equal(got, ref)


def test_slot_mapping_max_vblocks_bound(device):
    table = np.arange(12, dtype=np.int32).reshape(2, 6)
    positions = np.arange(0, 96, 5, dtype=np.int64)
    reqs = np.zeros_like(positions, dtype=np.int32)
    got = dcp.dcp_slot_mapping(torch.from_numpy(positions).to(device), torch.from_numpy(reqs).to(device),
                               torch.from_numpy(table).to(device), 4, 2, 2, max_vblocks=3).cpu().numpy()
    ref = olay.slot_mapping(positions, reqs, table, 4, 2, 2, max_vblocks=3)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# LSE merge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R,with_sink,out,B,H,Dv,offset", [
    (1, False, torch.float32, 3, 16, 72, 0), (2, True, torch.float32, 3, 16, 72, 0),
    (8, True, torch.bfloat16, 3, 16, 72, 0), (8, False, torch.bfloat16, 3, 16, 72, 0),
    (5, True, torch.float32, 3, 16, 72, 0), (64, False, torch.float32, 3, 16, 72, 0),
    # odd width (one value per thread), a width past one block of threads, and
    # rows that start off the 16-byte boundary (output and parts): scalar path
    (3, True, torch.bfloat16, 2, 5, 37, 0), (9, True, torch.float32, 2, 3, 1100, 0),
    (8, True, torch.float32, 2, 7, 128, 1), (8, False, torch.bfloat16, 2, 7, 128, 1),
    # the decode workloads' widths over many rows; more parts than one load batch
    (8, True, torch.bfloat16, 40, 64, 128, 0), (8, True, torch.bfloat16, 5, 128, 512, 0),
    (17, False, torch.float32, 6, 32, 512, 0), (12, True, torch.float32, 4, 3, 4, 0),
])
def test_lse_merge(device, R, with_sink, out, B, H, Dv, offset):
    rng = np.random.default_rng(R * 10 + with_sink + Dv)
    po = rng.standard_normal((R, B, H, Dv)).astype(np.float32)
    pl = (rng.standard_normal((R, B, H)) * 4).astype(np.float32)
    pl[rng.random((R, B, H)) < 0.3] = -np.inf                 # empty shards
    pl[:, 0, 0] = -np.inf                                      # an all-empty head
    po[np.isneginf(pl)] = 0.0
    sink = (rng.standard_normal(H) + 1).astype(np.float32) if with_sink else None
    # offset = 1: the part and output buffers start one element into an allocation
    po_dev = torch.empty(po.size + offset, dtype=torch.float32, device=device)[offset:].view(R, B, H, Dv)
    po_dev.copy_(torch.from_numpy(po))
    out_dev = torch.full(((B * H * Dv) + offset,), float("nan"), dtype=out, device=device)[offset:].view(B, H, Dv)
    o, lse = dcp.dcp_lse_merge(po_dev, torch.from_numpy(pl).to(device),
                               sink=None if sink is None else torch.from_numpy(sink).to(device), out_dtype=out,
                               out_o=out_dev)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        ro, rl = oatt.lse_merge(po[:, b], pl[:, b], sink)
        tol = dict(max_abs=1e-5 if out == torch.float32 else 2e-2, row_rel=1e-5, lse=1e-5)
        check_rows(o[b], ro, tol, f"merge b={b}", out_bf16=(out == torch.bfloat16))
        check_lse(lse[b], rl, tol, f"merge lse b={b}")


# ---------------------------------------------------------------------------
# partial attention + merge, reduced sizes with the workloads' geometry
# ---------------------------------------------------------------------------
SMALL = {
    "gqa_fp32_tiny": [None],
    "gqa_bf16_32k": [[1, 15, 16, 17, 31, 32, 33, 100, 257, 1000, 4099, 0]],
    "gqa_fp8_binned": [[1, 63, 64, 65, 511, 512, 513, 3000, 0, 10000, 129, 2]],
    "mla_bf16_bimodal": [[1, 31, 32, 33, 63, 64, 65, 700, 0, 2000, 4097]],
    "mla_bf16_longtail_sink": [[1, 5, 37, 600, 1500, 2049]],
}


def _algos(name):
    return [GEN] if name == "gqa_fp32_tiny" else [GEN, FAST]


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_small(device, name):
    w = get_workload(name)
    for lens in SMALL[name]:
        case = make_case(w, device=device, seq_lens=lens)
        inp = DeviceInputs(case, device)
        for algo in _algos(name):
            res = inp.run(algo=algo)
            check_against_oracle(inp, res)


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("scale", [0.0, -0.06])
def test_nonpositive_softmax_scale(device, name, scale):
    """A zero scale gives every cached token the same weight (the mean of V); a
    negative one favours the lowest scores. Every shard has a ragged tail, so
    the kernels' tail masks meet both."""
    import dataclasses
    w = dataclasses.replace(get_workload(name), scale_override=scale)
    case = make_case(w, device=device, seq_lens=[1, 37, 600, 2049, 0] if name != "gqa_fp32_tiny" else None)
    inp = DeviceInputs(case, device)
    for algo in _algos(name):
        check_against_oracle(inp, inp.run(algo=algo))


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_bimodal", "mla_bf16_longtail_sink"])
@pytest.mark.parametrize("bs,interleave", [(16, 1), (16, 16), (32, 8), (48, 16), (128, 64), (256, 1)])
def test_block_sizes(device, name, bs, interleave):
    """The MFMA kernels at block sizes other than the workloads' (any multiple
    of 16): tiles that span several blocks (16- and 32-token blocks), blocks
    whose size is not a power of two (48), and large blocks, with needles at
    block boundaries so that a misplaced block shows."""
    import dataclasses
    w = dataclasses.replace(get_workload(name), block_size=bs, interleave=interleave)
    case = make_case(w, device=device, seq_lens=[1, 17, 300, 2049, 0, 777], needles=3, needle_logit=20.0)
    inp = DeviceInputs(case, device)
    for algo in (GEN, FAST):
        check_against_oracle(inp, inp.run(algo=algo))


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_longtail_sink"])
def test_rank_subsets(device, name):
    """One GPU computing only its own rank(s), as a per-GPU deployment would."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[70, 1, 300, 2000, 0])
    inp = DeviceInputs(case, device)
    for algo in _algos(name):
        for rb, rc in [(0, 1), (1, 2), (inp.D - 1, 1)]:
            res = inp.run(algo=algo, rank_begin=rb, rank_count=rc)
            check_against_oracle(inp, res, rank_begin=rb)


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_bimodal"])
def test_invariance_over_dcp_and_interleave(device, name):
    """The merged result does not depend on dcp_size or the interleave size."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[777, 64, 5000, 1])
    outs = []
    bs = w.block_size
    for D, I in [(1, 1), (2, 1), (3, bs), (4, bs // 2), (8, bs), (8, 1)]:
        inp = DeviceInputs(case, device, dcp_size=D, interleave=I)
        res = inp.run(algo=FAST)
        check_against_oracle(inp, res, check_parts=False)
        outs.append(res[2].float().cpu().numpy())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


@pytest.mark.parametrize("name", ["gqa_fp8_binned", "gqa_bf16_32k", "mla_bf16_bimodal"])
def test_all_empty_batch(device, name):
    """No local token anywhere: no worker has a tile, and the combine writes
    every row from its empty-group pass."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[0, 0, 0])
    inp = DeviceInputs(case, device)
    for algo in (GEN, FAST):
        po, pl, o, lse = inp.run(algo=algo)
        assert torch.all(po == 0) and torch.all(torch.isneginf(pl))
        assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("name", ["gqa_fp8_binned", "mla_bf16_bimodal"])
def test_many_pairs_per_thread_chunk(device, name):
    """2,100 requests x 8 ranks = 16,800 (rank, request) pairs: the attention
    kernel's split search gives each of its 256 threads a chunk of 66 pairs
    (nine rounds of batched length loads), and a wavefront rescans the chunk
    holding its first tile in two rounds of 64. Short and zero lengths leave
    many ranks empty, so the combine's empty-group pass writes many rows.
    Every request is checked."""
    w = get_workload(name)
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 200, size=2100)
    lens[rng.random(2100) < 0.2] = 0
    case = make_case(w, device=device, seq_lens=[int(x) for x in lens])
    inp = DeviceInputs(case, device)
    check_against_oracle(inp, inp.run(algo=FAST))


def test_token_major_v_layout_uses_generic(device):
    w = get_workload("gqa_bf16_32k")
    case = make_case(w, device=device, seq_lens=[100, 33])
    inp = DeviceInputs(case, device, v_layout="token_major")
    check_against_oracle(inp, inp.run(algo=dcp.DCP_ALGO_AUTO))
    with pytest.raises(dcp.DcpError):
        inp.run(algo=FAST)


def test_fp8_codes_exhaustive(device):
    """Every finite e4m3 code, through the value path with one token per
    request (weight exactly 1): the partial output is code * v_scale exactly."""
    w = get_workload("gqa_fp8_binned")
    case = make_case(w, device=device, seq_lens=[1, 1])
    codes = np.arange(256, dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    for b in range(2):
        v = np.tile(codes[128 * b:128 * (b + 1)], (1, w.num_kv_heads, 1))
        case.v[b] = torch.from_numpy(v).to(device).view(torch.float8_e4m3fn)
    inp = DeviceInputs(case, device)
    tab = ofmt.e4m3fn_table()
    for algo in (GEN, FAST):
        po = inp.run(algo=algo)[0].cpu().numpy()           # [R, B, Hq, Dv]
        for b in range(2):
            owner = 0                                        # token 0 lives on rank 0
            for h in range(w.num_q_heads):
                ref = tab[codes[128 * b:128 * (b + 1)]] * np.float64(case.v_scale[h // w.group])
                np.testing.assert_allclose(po[owner, b, h], ref, rtol=2e-7, atol=0)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------
def test_full_gqa_bf16_32k_all_requests(device):
    w = get_workload("gqa_bf16_32k")
    case = make_case(w, device=device)
    inp = DeviceInputs(case, device)
    check_against_oracle(inp, inp.run(algo=FAST))


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_bimodal", "mla_bf16_longtail_sink"])
def test_large_logit_needles(device, name):
    """Needle keys scored ~120 above the rest late in the sequence: the MLA
    kernel's per-piece reference max is outgrown and the piece is replayed;
    the GQA kernel rescales. The output must follow the needles."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[3000, 129, 5000], needles=2, needle_logit=120.0)
    inp = DeviceInputs(case, device)
    for algo in _algos(name):
        check_against_oracle(inp, inp.run(algo=algo))


def test_mla_replay_in_later_unit(device):
    """Many short requests (about four tiles per rank), each with a needle
    scored ~120 above the rest at its last token: stream-K workers span many
    units, and pieces several units past a worker's first one outgrow their
    reference max and are replayed. The replay restarts the DMA walker there."""
    w = get_workload("mla_bf16_bimodal")
    lens = [1000 + 37 * (b % 7) for b in range(80)]
    case = make_case(w, device=device, seq_lens=lens, needles=1, needle_logit=120.0)
    inp = DeviceInputs(case, device)
    check_against_oracle(inp, inp.run(algo=FAST), requests=list(range(0, 80, 9)))


@pytest.mark.parametrize("name", ["gqa_bf16_32k", "gqa_fp8_binned", "mla_bf16_bimodal"])
def test_moderate_needles(device, name):
    """Needles at logit ~20 on every rank: a misplaced or dropped block shows
    an error of order one in the needle heads."""
    w = get_workload(name)
    case = make_case(w, device=device, seq_lens=[4000, 700, 65, 9000], needles=6, needle_logit=20.0)
    inp = DeviceInputs(case, device)
    for algo in _algos(name):
        check_against_oracle(inp, inp.run(algo=algo))


@pytest.mark.parametrize("name,lens", [("gqa_fp8_binned", [3000, 129, 7000, 1]),
                                       ("gqa_bf16_32k", [900, 2100, 5]),
                                       ("mla_bf16_bimodal", [3000, 650, 9000])])
def test_partials_into_unaligned_outputs(device, name, lens):
    """out_o and out_lse one float into their allocations (off the 16-byte
    grid): the MFMA kernels and the split combine (element-wise stores there)
    write the same partials, bit for bit, as into aligned outputs."""
    w = get_workload(name)
    inp = DeviceInputs(make_case(w, device=device, seq_lens=lens), device).prepare(algo=dcp.DCP_ALGO_FAST)
    inp.partial()
    torch.cuda.synchronize()
    ref_o, ref_l = inp.po.clone(), inp.pl.clone()
    po = torch.full((inp.po.numel() + 1,), float("nan"), device=device)[1:].view(inp.po.shape)
    pl = torch.full((inp.pl.numel() + 1,), float("nan"), device=device)[1:].view(inp.pl.shape)
    dcp.dcp_partial_decode_attn(inp.q, inp.kv, inp.block_table, inp.local_lens, inp.D, inp.rank_begin,
                                inp.rank_count, w.softmax_scale, po, pl, inp.ws, algo=dcp.DCP_ALGO_FAST)
    torch.cuda.synchronize()
    assert po.data_ptr() % 16 != 0
    assert torch.equal(po, ref_o) and torch.equal(pl, ref_l)
