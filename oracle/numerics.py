"""Exact decoding of the path's storage formats to float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

bf16 is the upper half of an IEEE binary32: widening its 16 bits to 32 and
reading them as a float is exact.  OCP fp8 e4m3fn ("E4M3" in the OCP 8-bit
floating point specification, v1.0) has 1 sign bit, 4 exponent bits with bias
7, 3 mantissa bits, subnormals at exponent field 0, no infinities and a single
NaN pattern per sign (exponent and mantissa all ones); its largest finite value
is 448.  The table below is written from that definition, not from any
library's conversion routine.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_value(byte: int) -> float:
    """Value of one OCP e4m3fn byte, from the format's definition."""
    s = (byte >> 7) & 1
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m / 8.0, 1 - 7)          # subnormal: 2^(1-bias) * 0.m
    else:
        mag = math.ldexp(1.0 + m / 8.0, e - 7)    # normal: 2^(e-bias) * 1.m
    return -mag if s else mag


E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def e4m3_bytes_to_f64(b: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """uint8 e4m3fn bytes -> float64 values times the per-tensor scale."""
    return E4M3_TABLE[np.asarray(b, dtype=np.uint8)] * float(scale)


def to_f64(x, scale: float = 1.0) -> np.ndarray:
    """A torch tensor or numpy array in f32 / bf16 / e4m3-bytes -> float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                return bf16_bits_to_f64(x.view(torch.int16).numpy().view(np.uint16))
            if x.dtype == torch.uint8:
                return e4m3_bytes_to_f64(x.numpy(), scale)
            if x.dtype == torch.float8_e4m3fn:
                return e4m3_bytes_to_f64(x.view(torch.uint8).numpy(), scale)
            return x.double().numpy() * float(scale)
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype == np.uint8:
        return e4m3_bytes_to_f64(a, scale)
    return a.astype(np.float64) * float(scale)


def round_to_bf16(x) -> np.ndarray:
    """The bf16 value nearest to each float64 (ties to the even significand),
    as float64.  bf16 keeps 8 significant bits and the exponent range of
    binary32: normal values from 2**-126, subnormal spacing 2**-133, largest
    finite (2 - 2**-7) * 2**127 (beyond it: infinity)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2**e, 0.5 <= |m| < 1
    y = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    tiny = np.abs(x) < 2.0 ** -126
    y = np.where(tiny, np.rint(x * 2.0 ** 133) * 2.0 ** -133, y)
    big = np.abs(y) > (2 - 2.0 ** -7) * 2.0 ** 127
    return np.where(big, np.copysign(np.inf, x), y)


def round_to_e4m3(x) -> np.ndarray:
    """The OCP e4m3fn value nearest to each float64 (ties to the even
    significand), saturated to +-448, as float64.  e4m3 keeps 4 significant
    bits: normal values 1.fff * 2**e for e in -6 .. 8 (largest 1.75 * 2**8 =
    448), subnormal spacing 2**-9 below 2**-6."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2**e, 0.5 <= |m| < 1
    y = np.ldexp(np.rint(np.ldexp(m, 4)), e - 4)
    tiny = np.abs(x) < 2.0 ** -6
    y = np.where(tiny, np.rint(x * 2.0 ** 9) * 2.0 ** -9, y)
    return np.clip(y, -448.0, 448.0)
