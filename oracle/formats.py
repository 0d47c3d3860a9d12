"""Exact float64 decoding of the stored KV-cache formats.

Test infrastructure: see the package docstring.

The stored representations are raw bit patterns held in NumPy arrays:

* fp32  - ``float32`` values (decoded as is);
* bf16  - ``uint16`` bit patterns, the top half of an IEEE binary32;
* fp8   - ``uint8`` codes in the OCP 8-bit floating point "E4M3" encoding
          (the variant without infinities, often called e4m3fn): 1 sign bit,
          4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
          subnormal, the all-ones code S.1111.111 is NaN, and the largest
          finite magnitude is 1.75 * 2**8 = 448.

The pages fix only "fp8 e4m3 KV with per-head fp32 scales"; the dequantised
value of a stored code c in KV head h is ``decode(c) * scale[h]``.
"""

import numpy as np

FP32, BF16, FP8_E4M3 = "fp32", "bf16", "fp8_e4m3"


def e4m3fn_value(code: int) -> float:
    """Value of one OCP E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        # subnormal: 0.man * 2**(1 - bias)
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3fn_table() -> np.ndarray:
    """All 256 code values as float64 (index = code)."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3_TABLE = e4m3fn_table()


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 widens into binary32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns decode to NaN
        return b.view(np.float32).astype(np.float64)


def decode(stored: np.ndarray, fmt: str) -> np.ndarray:
    """Stored representation -> float64, exactly."""
    if fmt == FP32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if fmt == BF16:
        return decode_bf16_bits(np.asarray(stored, dtype=np.uint16))
    if fmt == FP8_E4M3:
        return _E4M3_TABLE[np.asarray(stored, dtype=np.uint8)]
    raise ValueError(f"unknown stored format {fmt!r}")


def decode_kv(stored: np.ndarray, fmt: str, scale=None, head_axis: int = -2) -> np.ndarray:
    """Decode a KV tensor and, for fp8, multiply by the per-KV-head scale.

    ``stored`` has a KV-head axis (``head_axis``, default the second-to-last,
    as in ``[tokens, heads, dim]``); ``scale`` is ``[heads]`` float32 or None.
    """
    x = decode(stored, fmt)
    if scale is not None:
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        shape = [1] * x.ndim
        shape[head_axis] = s.shape[0]
        x = x * s.reshape(shape)
    return x
