"""Pins for the oracle's brute-force slot mapper and local lengths (CPU only).

Pinned against: the hand-worked example in tests/golden (derived from the
layout formulas of "Decode Context Parallel (DCP)", section "KV-cache layout"),
the closed form of the per-rank lengths derived independently below, the
layout's invariants, and the dcp_size = 1 special case (plain paged cache).
"""

import json
import os

import numpy as np
import pytest

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_worked_example.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: f"bs{c['block_size']}_d{c['dcp_size']}_i{c['interleave']}")
def test_worked_example(case):
    bs, D, I = case["block_size"], case["dcp_size"], case["interleave"]
    pos = np.asarray(case["positions"])
    assert list(layout.target_rank(pos, bs, D, I)) == case["target_rank"]
    slots = layout.slot_mapping(pos, np.zeros_like(pos), case["block_table"], bs, D, I)
    assert slots.tolist() == case["slots"]
    lens = layout.local_seq_lens([case["seq_len"]], bs, D, I)
    assert lens[0].tolist() == case["local_seq_lens"]


def _closed_form_lens(L, D, I):
    # Each full round of I*D tokens gives every rank I tokens; the remainder
    # fills ranks 0, 1, ... with up to I tokens each.
    full = L // (I * D)
    rem = L - full * I * D
    return [full * I + min(max(rem - r * I, 0), I) for r in range(D)]


SWEEP = [(bs, D, I) for bs in (1, 2, 4, 16, 64) for D in (1, 2, 3, 4, 8)
         for I in (1, 2, 4, 16, 64) if bs % I == 0]


@pytest.mark.parametrize("bs,D,I", SWEEP)
def test_local_lens_closed_form(bs, D, I):
    lens = [0, 1, 2, 3, 5, 17, 63, 64, 65, bs * D, bs * D + 1, 3 * bs * D - 1, 1000, 4097]
    got = layout.local_seq_lens(lens, bs, D, I)
    for L, row in zip(lens, got):
        assert row.tolist() == _closed_form_lens(L, D, I), (L, bs, D, I)


@pytest.mark.parametrize("bs,D,I", SWEEP)
def test_invariants(bs, D, I):
    L = 3 * bs * D + (bs * D) // 2 + 1
    nvb = (L + bs * D - 1) // (bs * D)
    rng = np.random.default_rng(bs * 100 + D * 10 + I)
    table = rng.permutation(nvb + 3)[:nvb][None, :]
    pos = np.arange(L)
    slots = layout.slot_mapping(pos, np.zeros(L, dtype=np.int64), table, bs, D, I)
    owners_ = (slots >= 0)
    # every token has exactly one owner, and it is rank (x // I) % D
    assert np.all(owners_.sum(axis=0) == 1)
    assert np.array_equal(np.argmax(owners_, axis=0), (pos // I) % D)
    for r in range(D):
        s = slots[r][slots[r] >= 0]
        assert np.unique(s).shape[0] == s.shape[0]            # unique per rank
        # slot lies in the block the table gives for the token's virtual block
        xs = pos[slots[r] >= 0]
        assert np.array_equal(s // bs, table[0, xs // (bs * D)])
        # rank-local order is ascending position: offsets count up inside a block
        for vb in range(nvb):
            sel = (xs // (bs * D)) == vb
            offs = s[sel] % bs
            assert np.array_equal(offs, np.arange(offs.shape[0]))
            if (vb + 1) * bs * D <= L:
                assert offs.shape[0] == bs                     # full block: bs tokens per rank
    lens = layout.local_seq_lens([L], bs, D, I)[0]
    assert lens.sum() == L
    assert lens.max() - lens.min() <= I
    assert lens[0] == lens.max()


def test_local_positions_match_slots():
    bs, D, I = 16, 4, 4
    L = 1000
    lp = layout.local_positions(L, bs, D, I)
    own = layout.owners(L, bs, D, I)
    nvb = (L + bs * D - 1) // (bs * D)
    table = np.arange(nvb)[None, :]
    slots = layout.slot_mapping(np.arange(L), np.zeros(L, dtype=np.int64), table, bs, D, I)
    assert np.array_equal(slots[own, np.arange(L)], lp)      # identity table: slot == local pos


def test_dcp1_is_plain_paged_cache():
    bs = 16
    L = 200
    table = np.array([[9, 3, 0, 7, 1, 12, 4, 2, 8, 5, 6, 11, 10]])
    slots = layout.slot_mapping(np.arange(L), np.zeros(L, dtype=np.int64), table, bs, 1, 1)
    x = np.arange(L)
    assert np.array_equal(slots[0], table[0, x // bs] * bs + x % bs)


def test_masked_and_out_of_range():
    bs, D, I = 4, 2, 1
    table = np.array([[3, -1], [0, 1]])
    pos = np.array([-1, 0, 8, 9, 20, 1, 9])
    req = np.array([0, 0, 0, 0, 1, 2, -1])
    slots = layout.slot_mapping(pos, req, table, bs, D, I)
    assert slots[:, 0].tolist() == [-1, -1]      # negative position
    assert slots[:, 1].tolist() == [12, -1]      # normal token
    assert slots[:, 2].tolist() == [-1, -1]      # block id -1
    assert slots[:, 4].tolist() == [-1, -1]      # virtual block past the table
    assert slots[:, 5].tolist() == [-1, -1]      # request index past the table
    assert slots[:, 6].tolist() == [-1, -1]      # negative request index


def test_constraint_rejected():
    # block_size % interleave != 0 would give ranks unequal shares of a virtual
    # block (bs=4, D=2, I=3: 5 and 3 tokens), which the layout forbids.
    with pytest.raises(ValueError):
        layout.in_block_offsets(4, 2, 3)
    with pytest.raises(ValueError):
        layout.local_seq_lens([10], 4, 2, 3)
    own = layout.target_rank(np.arange(8), 4, 2, 3)
    assert np.bincount(own, minlength=2).tolist() == [5, 3]


def test_planted_mistake_is_caught(monkeypatch):
    # A plausible slip (interleave applied after the modulo by dcp_size) must
    # fail the worked example.
    def wrong(x, block_size, dcp_size, interleave):
        return (x % (block_size * dcp_size)) % dcp_size // interleave

    monkeypatch.setattr(layout, "target_rank", wrong)
    case = _golden_cases()[0]
    pos = np.asarray(case["positions"])
    with pytest.raises(AssertionError):
        assert list(layout.target_rank(pos, case["block_size"], case["dcp_size"],
                                       case["interleave"])) == case["target_rank"]
