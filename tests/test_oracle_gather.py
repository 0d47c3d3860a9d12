"""Pins for the oracle's context gather (CPU only).

Pinned against: the round trip with the oracle's cache write (rows written at
their slots come back in request order, bit for bit, for every layout and
stored format), the hand-worked slot-mapping example in tests/golden (which
pool slot each gathered row comes from), dcp_size = 1 (a plain paged cache
read in position order), and zero rows for unmapped positions.
"""

import json
import os

import numpy as np
import pytest

from oracle import cache, formats, gather, layout


@pytest.mark.parametrize("bs,D,I", [(4, 2, 2), (16, 4, 1), (16, 3, 16), (8, 8, 4), (2, 1, 1), (64, 8, 64)])
@pytest.mark.parametrize("fmt", [formats.FP32, formats.BF16, formats.FP8_E4M3])
def test_round_trip_with_cache_write(bs, D, I, fmt):
    rng = np.random.default_rng(bs * 31 + D * 7 + I)
    lens = np.array([1, bs * D - 1, 3 * bs * D + 5, 0, 70], dtype=np.int64)
    span = bs * D
    nvb = [(int(n) + span - 1) // span for n in lens]
    N = sum(nvb) + 2
    perm = rng.permutation(N).astype(np.int32)
    table = np.full((len(lens), max(nvb)), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nvb):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    H, Dk, Dv = 2, 8, 16
    T = int(lens.sum())
    k_new = rng.standard_normal((T, H, Dk)).astype(np.float32)
    v_new = rng.standard_normal((T, H, Dv)).astype(np.float32)
    scale = np.array([0.3, 1.7], dtype=np.float32)
    dt = {formats.FP32: np.float32, formats.BF16: np.uint16, formats.FP8_E4M3: np.uint8}[fmt]
    kp = np.zeros((D, N, H, bs, Dk), dtype=dt)
    vp = np.zeros((D, N, H, Dv, bs), dtype=dt)
    positions = np.concatenate([np.arange(n) for n in lens])
    reqs = np.concatenate([np.full(n, b) for b, n in enumerate(lens)])
    slots = layout.slot_mapping(positions, reqs, table, bs, D, I)
    cache.cache_write(kp, vp, k_new, v_new, slots, bs, fmt, scale, scale)
    gk, gv = gather.gather_context(kp, vp, table, lens, bs, D, I)
    assert np.array_equal(gk, cache.store_values(k_new, fmt, scale))
    assert np.array_equal(gv, cache.store_values(v_new, fmt, scale))


def test_rows_come_from_the_worked_example_slots():
    with open(os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_worked_example.json")) as f:
        ex = json.load(f)["cases"][0]
    bs, D, I = ex["block_size"], ex["dcp_size"], ex["interleave"]
    table = np.array(ex["block_table"], dtype=np.int32)
    L = len(ex["slots"][0])
    kp = np.arange(D * 8 * bs, dtype=np.float32).reshape(D, 8, 1, bs, 1)    # value = its own flat index
    gk, _ = gather.gather_context(kp, None, table, [L], bs, D, I)
    for x in range(L):
        owner = [r for r in range(D) if ex["slots"][r][x] >= 0][0]
        s = ex["slots"][owner][x]
        assert gk[x, 0, 0] == (owner * 8 + s // bs) * bs + s % bs


def test_single_rank_is_a_plain_paged_read():
    bs, L = 4, 11
    table = np.array([[3, 0, 2]], dtype=np.int32)
    kp = np.random.default_rng(0).standard_normal((1, 4, 1, bs, 3)).astype(np.float32)
    gk, _ = gather.gather_context(kp, None, table, [L], bs, 1, 1)
    for x in range(L):
        assert np.array_equal(gk[x, 0], kp[0, table[0, x // bs], 0, x % bs])


def test_unmapped_positions_are_zero():
    kp = np.ones((2, 4, 1, 4, 2), dtype=np.float32)
    table = np.array([[1, -1]], dtype=np.int32)                        # second virtual block unallocated
    gk, _ = gather.gather_context(kp, None, table, [12], 4, 2, 1)
    assert np.all(gk[:8] == 1) and np.all(gk[8:] == 0)
    gk, _ = gather.gather_context(kp, None, table, [12], 4, 2, 1, max_vblocks=1)
    assert np.all(gk[8:] == 0)
