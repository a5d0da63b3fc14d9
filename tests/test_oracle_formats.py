"""Pins of the oracle's scalar codecs against independent decoders and the OCP tables."""
import math

import numpy as np
import pytest
import torch

from oracle import formats


# OCP Microscaling Formats v1.0, FP4 E2M1 value table (magnitudes of codes 0..7).
OCP_E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_matches_ocp_table():
    for c in range(16):
        v = formats.e2m1_value(c)
        mag = OCP_E2M1_MAGNITUDES[c & 7]
        assert abs(v) == mag
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)
    np.testing.assert_array_equal(formats.decode_e2m1(np.arange(16)), formats.E2M1_TABLE)


def test_e4m3_exhaustive_against_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = formats.e4m3_value(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), hex(b)
        else:
            assert v == ref[b], hex(b)
            assert math.copysign(1.0, v) == math.copysign(1.0, ref[b])


def test_e4m3_landmarks():
    # OCP 8-bit FP spec: max normal 448, min normal 2^-6, min subnormal 2^-9, one NaN per sign
    assert formats.e4m3_value(0x7E) == 448.0
    assert formats.e4m3_value(0x08) == 2.0 ** -6
    assert formats.e4m3_value(0x01) == 2.0 ** -9
    assert formats.e4m3_value(0x38) == 1.0
    assert math.isnan(formats.e4m3_value(0x7F)) and math.isnan(formats.e4m3_value(0xFF))
    with pytest.raises(ValueError):
        formats.decode_e4m3(np.array([0x7F], dtype=np.uint8))


def test_bf16_exhaustive_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    for b in (0x3F80, 0xC000, 0x0001, 0x7F7F):
        assert formats.bf16_value(b) == got[b]
