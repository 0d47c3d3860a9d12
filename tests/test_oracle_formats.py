"""Pins for the oracle's stored-format decoding (CPU only).

Pinned against torch's own float8_e4m3fn and bfloat16 conversions (library
routines, independent of the oracle) and against values fixed by the OCP E4M3
definition.
"""

import numpy as np
import torch

from oracle import formats


def test_e4m3fn_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = formats.e4m3fn_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert np.array_equal(ref[~nan], tab[~nan])


def test_e4m3fn_definition_values():
    v = formats.e4m3fn_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0
    assert v(0x38) == 1.0                      # exponent 7 = bias, mantissa 0
    assert v(0x7E) == 448.0                    # largest finite
    assert v(0xFE) == -448.0
    assert v(0x01) == 2.0 ** -9                # smallest subnormal
    assert v(0x08) == 2.0 ** -6                # smallest normal
    assert v(0x07) == 7 * 2.0 ** -9            # largest subnormal
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x78) == 256.0                    # no infinity: exponent 15 is finite
    # exactly 2 NaN codes, every other code finite
    tab = formats.e4m3fn_table()
    assert np.isnan(tab).sum() == 2


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.decode(bits, formats.BF16), x.to(torch.float64).numpy())


def test_decode_kv_scales_per_head():
    codes = np.full((3, 2, 4), 0x38, dtype=np.uint8)          # all 1.0
    out = formats.decode_kv(codes, formats.FP8_E4M3, scale=np.array([0.5, 3.0], np.float32))
    assert np.all(out[:, 0, :] == 0.5) and np.all(out[:, 1, :] == 3.0)
