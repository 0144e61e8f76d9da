"""Test-side helpers that are independent of both the oracle and the library.

`bf16_rne` rounds a double to bf16 by integer manipulation of its IEEE-754
bits (a different algorithm from the oracle's grid-scaling rounding), so tests
that expect a bf16 result do not lean on the code under test.
"""
import math
import struct

import numpy as np


def bf16_rne(v: float) -> int:
    """Nearest bf16 (ties to even) of a double, from its bit pattern."""
    bits = struct.unpack("<Q", struct.pack("<d", float(v)))[0]
    sign = (bits >> 63) & 1
    exp = (bits >> 52) & 0x7FF
    frac = bits & ((1 << 52) - 1)
    if exp == 0x7FF:
        return (sign << 15) | (0x7FC0 if frac else 0x7F80)
    if exp == 0:  # double subnormals are far below bf16's range
        return sign << 15
    e = exp - 1023
    mant = (1 << 52) | frac          # 53-bit significand, value = mant * 2^(e-52)
    if e >= -126:
        shift = 52 - 7               # keep 8 significant bits
        bexp = e + 127
    else:                            # bf16 subnormal: spacing 2^-133
        shift = 52 - 7 + (-126 - e)
        bexp = 0
    if shift >= 64:
        return sign << 15
    keep = mant >> shift
    rem = mant & ((1 << shift) - 1)
    half = 1 << (shift - 1)
    if rem > half or (rem == half and (keep & 1)):
        keep += 1
    if bexp == 0:
        # subnormal: keep is the 7-bit fraction (may carry into the smallest normal)
        return (sign << 15) | keep
    if keep == (1 << 8):             # carried into the next binade
        keep >>= 1
        bexp += 1
    if bexp >= 0xFF:
        return (sign << 15) | 0x7F80
    return (sign << 15) | (bexp << 7) | (keep & 0x7F)


def bf16_val(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


def f32(v: float) -> float:
    return float(np.float32(v))


def rel_l2_rows(got: np.ndarray, want: np.ndarray) -> float:
    """max over rows of ||got - want||_2 / ||want||_2 (bf16 bit arrays in)."""
    g = (np.asarray(got, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = (np.asarray(want, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g = g.reshape(-1, g.shape[-1])
    w = w.reshape(-1, w.shape[-1])
    num = np.linalg.norm(g - w, axis=1)
    den = np.maximum(np.linalg.norm(w, axis=1), 1e-30)
    return float(np.max(num / den)) if g.shape[0] else 0.0
