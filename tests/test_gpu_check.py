"""dcp_check_block_table: the count of in-use block-table entries that are
missing or outside the pool, against a plain count of the same definition
(request b of length L uses virtual blocks 0 .. ceil(L / (block_size *
dcp_size)) - 1; the layout's virtual block spans block_size * dcp_size
positions)."""

import numpy as np
import pytest
import torch

import sequence_sharded_paged_amd as dcp
from workloads import WORKLOADS
from workloads.generate import make_block_table, sample_lengths

pytestmark = pytest.mark.gpu


def _expected(table, lens, max_vblocks, bs, D, num_blocks):
    bad = 0
    for b, L in enumerate(lens):
        need = -(-max(int(L), 0) // (bs * D))
        for vb in range(need):
            if vb >= max_vblocks or not (0 <= table[b, vb] < num_blocks):
                bad += 1
    return bad


def _run(device, table, lens, bs, D, num_blocks, max_vblocks=None):
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)
    s = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(device)
    out = dcp.dcp_check_block_table(t, s, bs, D, num_blocks, max_vblocks=max_vblocks)
    return int(out.item())


def test_valid_and_corrupted_tables(device):
    rng = np.random.default_rng(7)
    bs, D, N = 16, 4, 500
    lens = [0, 1, 64, 65, 1000, 5000, -3]
    maxv = 80
    table = rng.integers(0, N, size=(len(lens), 96)).astype(np.int32)
    assert _run(device, table, lens, bs, D, N, maxv) == 0
    bad = table.copy()
    bad[2, 0] = -1                   # in use
    bad[4, 3] = N                    # in use, one past the pool
    bad[5, 78] = 2 ** 30             # in use, last needed entry of request 5
    bad[1, 1] = -9                   # beyond request 1's single block: not counted
    bad[3, 50] = N + 7               # beyond request 3's two blocks: not counted
    bad[0, 0] = -1                   # empty request: not counted
    bad[6, 0] = -1                   # negative length reads as empty
    got = _run(device, bad, lens, bs, D, N, maxv)
    assert got == _expected(bad, lens, maxv, bs, D, N) == 3
    # a table narrower than the lengths need: the missing entries count
    got = _run(device, table, lens, bs, D, N, 60)
    assert got == _expected(table, lens, 60, bs, D, N) == 79 - 60


def test_empty_batch_clears_the_count(device):
    out = torch.full((1,), 123, dtype=torch.int32, device=device)
    t = torch.zeros((0, 4), dtype=torch.int32, device=device)
    s = torch.zeros((0,), dtype=torch.int32, device=device)
    dcp.dcp_check_block_table(t, s, 16, 2, 10, out=out)
    assert int(out.item()) == 0


@pytest.mark.parametrize("name", ["gqa_fp8_binned", "mla_bf16_longtail_sink"])
def test_workload_tables_are_valid(device, name):
    w = WORKLOADS[name]
    lens = sample_lengths(w)
    table, nblocks = make_block_table(w, lens, 0)
    assert _run(device, table, lens, w.block_size, w.dcp_size, nblocks) == 0
    assert _run(device, table, lens, w.block_size, w.dcp_size, nblocks - 1) == _expected(
        table, lens, table.shape[1], w.block_size, w.dcp_size, nblocks - 1)
