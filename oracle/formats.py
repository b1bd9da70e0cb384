"""Decoders for the storage formats of Q, K and V (oracle; test infrastructure).

bf16: the upper 16 bits of an IEEE-754 binary32 value.
e4m3: the OCP 8-bit floating-point format with 4 exponent bits (bias 7) and 3
mantissa bits, no infinities, NaN at S.1111.111, largest finite value 448.  The
pages name FP8 storage of the KV data for long inputs (novita.ai blog,
"Revolutionizing LLM inference ...", sections "Proprietary FP8 quantization
scheme" and "Inference process optimization"), with scaling factors; they do not
fix the bit layout, so the OCP e4m3 layout is taken as the plainest reading.

Both decoders are written from the format definitions, element by element,
with no lookup table shared with any other code.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP e4m3 codes (uint8) -> float64, exactly.

    value = (-1)^s * 2^(e-7) * (1 + m/8)   for exponent field e in 1..15
          = (-1)^s * 2^(-6)  * (m/8)       for e = 0 (subnormals and zero)
    except code S.1111.111, which is NaN.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = sign * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, v)
