"""Bit-exact decoders for the stored formats, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E4M3FN ("FN": finite, no infinities), the FP8 format that gfx950 uses with a
largest finite value of 448 (sglang#27745 page, "Code analysis 1: FP8
quantisation", runtime architecture detection):
    code = S EEEE MMM, exponent bias 7
    E == 0        : (-1)^S * 2^-6 * M/8               (zero and subnormals)
    E >= 1        : (-1)^S * 2^(E-7) * (1 + M/8)
    E == 15, M==7 : NaN (no infinity exists)
E2M1 (the NVFP4 element format): code = S EE M, exponent bias 1
    E == 0        : (-1)^S * M/2                      (0 or 0.5)
    E >= 1        : (-1)^S * 2^(E-1) * (1 + M/2)      (1, 1.5, 2, 3, 4, 6)
Packed FP4: element 2j is the low nibble of byte j, element 2j+1 the high
nibble (reading: the pages print no nibble order; the low-byte-first packing
of two FP8 codes on the sglang#27745 page is followed).  The order cannot
change a GEMM result as long as A and B use the same one.
BF16: FP32 -> BF16 round to nearest, ties to even (reading: the pages only
say "BF16 output").
"""
from __future__ import annotations

import numpy as np


def decode_e4m3fn(codes) -> np.ndarray:
    """E4M3FN codes (uint8) -> float64 values; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    S = (c >> 7) & 1
    E = (c >> 3) & 0xF
    M = c & 0x7
    sub = np.ldexp(M / 8.0, -6)
    nrm = np.ldexp(1.0 + M / 8.0, E - 7)
    mag = np.where(E == 0, sub, nrm)
    out = np.where(S == 1, -mag, mag)
    out = np.where((E == 15) & (M == 7), np.nan, out)
    return out.astype(np.float64)


def decode_e2m1(nibbles) -> np.ndarray:
    """E2M1 codes (0..15) -> float64 values."""
    c = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 0xF
    S = (c >> 3) & 1
    E = (c >> 1) & 0x3
    M = c & 0x1
    mag = np.where(E == 0, M / 2.0, np.ldexp(1.0 + M / 2.0, E - 1))
    return np.where(S == 1, -mag, mag).astype(np.float64)


def unpack_e2m1(packed) -> np.ndarray:
    """Packed FP4 bytes [..., K/2] -> E2M1 codes [..., K] (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def bf16_rne_bits(x) -> np.ndarray:
    """Round float64 values to BF16 (8 significant bits, RNE) -> uint16 bits.

    The value is first rounded to FP32 the way the kernel's FP32 accumulator
    holds it, then to BF16 with ties to even; NaN maps to the canonical
    quiet NaN 0x7FC0.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), out).astype(np.uint16)


def bf16_bits_to_float(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
