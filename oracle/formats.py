"""Scalar codecs, written from the public format definitions (test infrastructure).

* FP4 E2M1 (OCP Microscaling Formats v1.0): sign bit, 2 exponent bits with bias 1,
  1 mantissa bit; exponent field 0 is subnormal (value 0.5*m); no inf or NaN.
* FP8 E4M3 "FN" (OCP 8-bit Floating Point v1.0): sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 is subnormal (2^-6 * m/8); the code
  with all exponent and mantissa bits set is NaN; there is no infinity.
* bf16: the high half of an IEEE-754 binary32 bit pattern.

The pages fix only "NVFP4 with FP8 block scales" (page "GLM 5.3 Testing: HBM
Expert Allocation", section "What the slot cache is"); the exact variant (E2M1
values, E4M3 per-16 scales, an fp32 global scale) is the plain NVFP4 reading.
"""
import struct

import numpy as np


def e2m1_value(code: int) -> float:
    code = int(code) & 0xF
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e4m3_value(byte: int) -> float:
    byte = int(byte) & 0xFF
    s, e, m = byte >> 7, (byte >> 3) & 0xF, byte & 7
    if e == 0xF and m == 7:
        return float("nan")
    mag = 2.0 ** -6 * (m / 8.0) if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def decode_e2m1(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def decode_e4m3(bytes_, allow_nan: bool = False) -> np.ndarray:
    v = E4M3_TABLE[np.asarray(bytes_, dtype=np.uint8)]
    if not allow_nan and np.isnan(v).any():
        raise ValueError("E4M3 NaN code in a block scale")
    return v


def decode_bf16(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)
