"""Pins for the oracle's KV-cache write (CPU only).

Pinned against: the E4M3 code table's own values (every finite code must come
back unchanged, exact midpoints must go to the even code, the format's largest
finite value bounds everything), hand-worked values, an exhaustive brute-force
nearest search over all 65,536 bf16 patterns (independent of the oracle's
two-candidate rounding), and the hand-worked slot-mapping example in
tests/golden for where each written row lands.
"""

import json
import os

import numpy as np
import pytest

from oracle import cache, formats

TABLE = formats.e4m3fn_table()
FINITE = [c for c in range(256) if not np.isnan(TABLE[c])]


def test_e4m3_every_finite_code_round_trips():
    vals = np.array([TABLE[c] for c in FINITE], dtype=np.float64)
    signs = np.array([bool(c & 0x80) for c in FINITE])
    x = np.where(signs, -np.abs(vals), np.abs(vals)).astype(np.float32)  # keeps -0.0 for 0x80
    assert list(cache.quantize_e4m3fn(x)) == FINITE


def test_e4m3_midpoints_go_to_even_code():
    pos = [c for c in range(0x7F)]  # non-negative finite codes in increasing value order
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((TABLE[a] + TABLE[b]) / 2)  # exact in fp32 (4 significant bits)
        assert float(mid) == (TABLE[a] + TABLE[b]) / 2
        even = a if a % 2 == 0 else b
        assert cache.quantize_e4m3fn(mid)[()] == even, (a, b)
        assert cache.quantize_e4m3fn(-mid)[()] == (even | 0x80), (a, b)
        above = np.nextafter(mid, np.float32(np.inf))
        below = np.nextafter(mid, np.float32(0))
        assert cache.quantize_e4m3fn(above)[()] == b
        assert cache.quantize_e4m3fn(below)[()] == a


def test_e4m3_hand_values_saturation_nan_zero():
    q = lambda v: int(cache.quantize_e4m3fn(np.float32(v))[()])
    assert q(1.0) == 0x38             # exponent field 7, mantissa 0
    assert q(-1.5) == 0xBC            # sign, exponent 7, mantissa 4
    assert q(2.0 ** -9) == 0x01       # smallest subnormal
    assert q(2.0 ** -10) == 0x00      # halfway to the smallest subnormal: ties to even (zero)
    assert q(3 * 2.0 ** -10) == 0x02  # halfway between codes 1 and 2 -> 2
    assert q(2.0 ** -6) == 0x08       # smallest normal
    assert q(448.0) == 0x7E
    assert q(464.0) == 0x7E           # past the largest finite value: saturates
    assert q(1e30) == 0x7E and q(-1e30) == 0xFE
    assert q(np.inf) == 0x7E and q(-np.inf) == 0xFE
    assert q(np.nan) == 0x7F
    assert q(0.0) == 0x00 and q(-0.0) == 0x80


def _bf16_brute(x):
    """Nearest bf16 pattern by scanning all 65,536 codes (ties: even code)."""
    codes = np.arange(65536, dtype=np.uint32)
    vals = formats.decode_bf16_bits(codes.astype(np.uint16))
    ok = np.isfinite(vals)
    out = []
    for v in np.asarray(x, dtype=np.float32).astype(np.float64):
        d = np.where(ok, np.abs(vals - v), np.inf)
        best = np.flatnonzero(d == d.min())
        best = [c for c in best if np.signbit(formats.decode_bf16_bits(np.uint16(c))) == np.signbit(v)] or list(best)
        even = [c for c in best if c % 2 == 0]
        out.append(int((even or best)[0]))
    return np.array(out, dtype=np.uint16)


def test_bf16_rounding_matches_brute_force():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(50) * 1e-38).astype(np.float32),      # subnormal range
        rng.uniform(-1e30, 1e30, 50).astype(np.float32),
    ])
    assert np.array_equal(cache.round_bf16_bits(x), _bf16_brute(x))


def test_bf16_round_trip_and_ties():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = formats.decode_bf16_bits(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(cache.round_bf16_bits(vals[fin].astype(np.float32)), codes[fin])
    r = lambda v: int(cache.round_bf16_bits(np.float32(v))[()])
    assert r(1.0 + 2.0 ** -8) == 0x3F80          # tie between 1.0 (even) and 1.0078125
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie between 0x3F81 and 0x3F82 -> even
    assert r(np.inf) == 0x7F80 and r(-np.inf) == 0xFF80
    assert np.isnan(formats.decode_bf16_bits(np.uint16(r(np.nan))))


def test_store_values_fp8_uses_the_head_scale():
    scale = np.array([0.5, 3.0], dtype=np.float32)
    codes = np.array([[0x38, 0x3C], [0x01, 0xC5]], dtype=np.uint8)          # [heads, dim]
    x = (TABLE[codes] * scale[:, None]).astype(np.float32)[None]             # exact products
    assert np.array_equal(cache.store_values(x, formats.FP8_E4M3, scale)[0], codes)


def test_cache_write_places_rows_by_the_worked_example():
    with open(os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_worked_example.json")) as f:
        ex = json.load(f)["cases"][0]
    bs, D = ex["block_size"], ex["dcp_size"]
    slots = np.array(ex["slots"], dtype=np.int64)
    T, H, Dk, Dv, N = slots.shape[1], 2, 3, 2, 8
    k_new = np.arange(T * H * Dk, dtype=np.float32).reshape(T, H, Dk) + 1
    v_new = -np.arange(T * H * Dv, dtype=np.float32).reshape(T, H, Dv) - 1
    k_pool = np.zeros((D, N, H, bs, Dk), dtype=np.float32)
    v_pool = np.zeros((D, N, H, Dv, bs), dtype=np.float32)
    cache.cache_write(k_pool, v_pool, k_new, v_new, slots, bs, formats.FP32)
    # token 8 -> rank 0, block 2, offset 0; token 11 -> rank 1, block 2, offset 1 (hand-worked)
    assert np.array_equal(k_pool[0, 2, :, 0, :], k_new[8])
    assert np.array_equal(v_pool[0, 2, :, :, 0], v_new[8])
    assert np.array_equal(k_pool[1, 2, :, 1, :], k_new[11])
    assert np.array_equal(v_pool[1, 5, :, :, 3], v_new[7])        # token 7: rank 1, slot 23
    written = sum(int((slots[r] >= 0).sum()) for r in range(D))
    assert written == T                                           # every token owned exactly once
    assert np.count_nonzero(k_pool) == T * H * Dk


def test_cache_write_skips_unowned_and_out_of_range_slots():
    k_pool = np.zeros((2, 2, 1, 4, 2), dtype=np.float32)
    slots = np.array([[-1, 8, 3], [2, -5, -1]], dtype=np.int64)     # 8 = 2 blocks x 4: out of range
    k_new = np.ones((3, 1, 2), dtype=np.float32)
    cache.cache_write(k_pool, None, k_new, None, slots, 4, formats.FP32)
    assert k_pool[0, 0, 0, 3].tolist() == [1.0, 1.0] and k_pool[1, 0, 0, 2].tolist() == [1.0, 1.0]
    assert np.count_nonzero(k_pool) == 4
