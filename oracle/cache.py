"""KV-cache write of new rows into the per-rank DCP pools (float64 / exact
integer reference).

Test infrastructure: see the package docstring.

Sources: "Decode Context Parallel (DCP)" (vLLM Ascend developer guide),
section "KV-cache layout" (each rank stores only its local shard, at the slot
the slot mapping gives); "DeepSeek V4.1 context parallelism" (TokenSpeed design
note), section "Cache ownership" (a write turns the virtual slot into the
owner's local slot and non-owners are masked). The pages fix the stored fp8
format only as "e4m3 with per-head fp32 scales"; the readings taken here:

* a stored fp8 code is the E4M3 (no-infinity) value nearest to the fp32
  quotient ``float32(x) / scale[h]``, ties to the even code, magnitudes past
  the largest finite value (448, infinities included) saturate to it, NaN
  stays NaN (code 0x7F), and zero keeps its sign;
* a stored bf16 value is the fp32 input rounded to nearest, ties to even;
* fp32 caches store the fp32 input as is;
* slots are ``[num_ranks, T]``; ``-1`` marks a rank that does not own token t
  and so does any value outside ``[0, num_blocks * block_size)``: nothing is
  written for it.

Pool layouts (the ones the attention kernels read): K ``[rank, block, head,
token, dim]``; GQA V ``[rank, block, head, dim, token]``; MLA has no V pool.
"""

import numpy as np

from . import formats

_E4M3 = formats.e4m3fn_table()
# Codes 0x00 .. 0x7E are the non-negative finite values in increasing order.
_POS_VALUES = _E4M3[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def quantize_e4m3fn(q) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8): nearest finite value, ties to the
    even code, saturating; NaN -> 0x7F; the sign goes to bit 7."""
    q = np.asarray(q, dtype=np.float32)
    mag = np.abs(q.astype(np.float64))
    sign = np.signbit(q)
    nan = np.isnan(q)
    mag = np.where(nan, 0.0, np.minimum(mag, _POS_VALUES[-1]))  # saturate (inf included)
    # neighbours below and above |q| in the table of non-negative values
    hi = np.searchsorted(_POS_VALUES, mag, side="left")          # first value >= |q|
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(sign, code | np.uint8(0x80), code)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


def round_bf16_bits(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest, ties to
    even; NaN stays a (quiet) NaN, infinities stay infinite."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):  # NaN inputs take the explicit branch below
        return _round_bf16_bits(x)


def _round_bf16_bits(x):
    bits = x.view(np.uint32).astype(np.uint64)
    down = (bits >> np.uint64(16)).astype(np.uint64)        # truncation toward zero (same sign)
    up = down + np.uint64(1)                                # next bf16 away from zero
    v = np.abs(x.astype(np.float64))
    v_down = np.abs(formats.decode_bf16_bits(down.astype(np.uint16)))
    # the value one bf16 step away from zero; past the largest finite bf16 the
    # step lands on 2**128 (the rounding threshold), not on the infinity code
    v_up = np.where((up & np.uint64(0x7FFF)) == np.uint64(0x7F80), 2.0 ** 128,
                    np.abs(formats.decode_bf16_bits((up & np.uint64(0xFFFF)).astype(np.uint16))))
    d_down = v - v_down
    d_up = v_up - v
    take_up = (d_up < d_down) | ((d_up == d_down) & (down % np.uint64(2) == np.uint64(1)))
    out = np.where(take_up, up, down).astype(np.uint64)
    nan = np.isnan(x)
    inf = np.isinf(x)
    out = np.where(inf, down, out)                          # inf truncates to inf exactly
    out = np.where(nan, (down | np.uint64(0x0040)), out)    # quiet NaN, sign kept
    return (out & np.uint64(0xFFFF)).astype(np.uint16)


def store_values(x, fmt: str, scale=None) -> np.ndarray:
    """fp32 input rows ``[..., heads, dim]`` -> stored representation in ``fmt``.
    For fp8, ``scale`` is ``[heads]`` float32 and the quotient is taken in fp32."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == formats.FP32:
        return x.copy()
    if fmt == formats.BF16:
        return round_bf16_bits(x)
    if fmt == formats.FP8_E4M3:
        s = np.asarray(scale, dtype=np.float32).reshape([1] * (x.ndim - 2) + [-1, 1])
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):  # IEEE results are wanted
            q = (x / s).astype(np.float32)
        return quantize_e4m3fn(q)
    raise ValueError(f"unknown stored format {fmt!r}")


def cache_write(k_pool, v_pool, k_new, v_new, slots, block_size: int, fmt: str, k_scale=None, v_scale=None):
    """Write new rows into the pools (in place) and return them.

    ``k_pool``: stored ``[R, N, H, block_size, Dk]``; ``v_pool``: stored
    ``[R, N, H, Dv, block_size]`` or None (MLA); ``k_new [T, H, Dk]``,
    ``v_new [T, H, Dv]`` fp32 (or None); ``slots [R, T]`` int64.
    """
    slots = np.asarray(slots, dtype=np.int64)
    R, N = k_pool.shape[0], k_pool.shape[1]
    k_st = store_values(k_new, fmt, k_scale)
    v_st = None if v_new is None else store_values(v_new, fmt, v_scale)
    for r in range(R):
        for t in range(slots.shape[1]):
            s = int(slots[r, t])
            if s < 0 or s >= N * block_size:
                continue
            blk, off = divmod(s, block_size)
            k_pool[r, blk, :, off, :] = k_st[t]
            if v_pool is not None and v_st is not None:
                v_pool[r, blk, :, :, off] = v_st[t]
    return k_pool, v_pool
