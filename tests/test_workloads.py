"""Host checks of the seeded input generators (CPU only)."""

import numpy as np
import pytest

from workloads import WORKLOADS, get_workload, make_case
from workloads.generate import make_block_table, sample_lengths


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_lengths_follow_the_laws(name):
    w = get_workload(name)
    lens = sample_lengths(w)
    assert lens.shape[0] == w.batch
    assert np.array_equal(lens, sample_lengths(w))          # deterministic
    lo = min(a for _, _, a, _ in w.lengths)
    hi = max(b for _, _, _, b in w.lengths)
    assert lens.min() >= lo and lens.max() <= hi
    for count, law, a, b in w.lengths:
        if len(w.lengths) > 1:
            assert count <= ((lens >= a) & (lens <= b)).sum()


def test_bin_counts():
    w = get_workload("gqa_fp8_binned")
    assert [c for c, *_ in w.lengths] == [46, 74, 115, 21]
    w = get_workload("mla_bf16_bimodal")
    assert [c for c, *_ in w.lengths] == [30, 34]


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_block_table_is_a_permutation(name):
    w = get_workload(name)
    lens = sample_lengths(w)
    table, nblk = make_block_table(w, lens)
    used = table[table >= 0]
    assert np.array_equal(np.sort(used), np.arange(nblk))
    span = w.block_size * w.dcp_size
    for b, L in enumerate(lens):
        n = (int(L) + span - 1) // span
        assert np.all(table[b, :n] >= 0) and np.all(table[b, n:] == -1)


def test_small_case_shapes_and_determinism():
    w = get_workload("gqa_fp32_tiny")
    c1, c2 = make_case(w), make_case(w)
    assert c1.seq_lens.tolist() == [37, 100]
    assert tuple(c1.q.shape) == (2, 8, 64)
    assert tuple(c1.k[1].shape) == (100, 2, 64) and tuple(c1.v[0].shape) == (37, 2, 64)
    assert all((a == b).all() for a, b in zip(c1.k, c2.k))
    w = get_workload("gqa_fp8_binned")
    c = make_case(w, seq_lens=[5, 70])
    assert str(c.k[0].dtype) == "torch.float8_e4m3fn" and c.k_scale.shape == (8,)
    assert len(set(c.k_scale.tolist())) == 8
    w = get_workload("mla_bf16_longtail_sink")
    c = make_case(w, seq_lens=[3, 9])
    assert c.v is None and c.sink.shape == (128,)
