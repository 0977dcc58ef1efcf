"""Oracle for the activation quantisers (the step before the GEMM).

TEST INFRASTRUCTURE ONLY (see the package docstring): used by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the GPU path.

What is computed (sglang#27745 page, "Code analysis 1: FP8 quantisation":
values are clamped to +-448, the E4M3FN maximum on gfx950, zero encodes to
code 0, and the code is sign | exponent << 3 | mantissa; the per-128 block
scales are the FP32 scales the flashinfer#7877 page names; the NVFP4 layout
is the one of the onnxruntime#29824 page's W4A4 path):

  FP8 1x128   for each row i and 128-wide K block kb of X (BF16 values):
                amax  = max |X[i, kb-block]|
                scale = amax / 448            (an all-zero block: 1.0)
                code  = E4M3FN(clamp(X / scale, -448, 448))
  NVFP4       g      = amax(X) / (6 * 448)    (all-zero X: 1.0)
              per row and 16-wide block: s = E4M3FN(clamp(bamax / (6 g), 448)),
                d = value(s) * g; code = E2M1(clamp(X / d, -6, 6)), 0 where d = 0;
              two codes per byte, element 2j in the low nibble of byte j.

Every arithmetic step that decides a code is taken in FP32 with IEEE
round-to-nearest-even (NumPy float32 scalar/array arithmetic), the precision
the GPU kernels decide in; the encoders round to the nearest representable
value, ties to the even code, by searching the format's value table, which
is built from the bit-field definitions in formats.py.

Parity status: pinned (tests/test_oracle_quant.py: exhaustive round trips of
every finite code, every midpoint between neighbouring values, saturation,
zero blocks, torch's float8_e4m3fn cast of clamped values, and reconstruction
of inputs built from codes and scales).
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e2m1, decode_e4m3fn

E4M3_MAX = np.float32(448.0)
E2M1_MAX = np.float32(6.0)


def _nearest_code(x, codes, values) -> np.ndarray:
    """Round each float32 in x to the code whose value is nearest (ties to
    the code with even mantissa LSB), given the non-negative finite codes and
    their values in increasing order; the sign is carried separately."""
    x = np.asarray(x, dtype=np.float32)
    neg = np.signbit(x)
    a = np.abs(x).astype(np.float64)  # exact: every float32 is a float64
    v = values.astype(np.float64)
    hi = np.clip(np.searchsorted(v, a, side="left"), 0, v.size - 1)
    lo = np.clip(hi - 1, 0, v.size - 1)
    d_lo = np.abs(a - v[lo])
    d_hi = np.abs(v[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    idx = np.where(pick_hi, hi, lo)
    return codes[idx], neg


def e4m3fn_round(x) -> np.ndarray:
    """float32 values (already within +-448) -> E4M3FN codes, round to
    nearest, ties to even; -0.0 and negatives below half the smallest
    subnormal keep the sign bit (code 0x80)."""
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: 0 .. 448, increasing
    values = decode_e4m3fn(codes)
    c, neg = _nearest_code(x, codes, values)
    return (c | np.where(neg, 0x80, 0x00)).astype(np.uint8)


def e2m1_round(x) -> np.ndarray:
    """float32 values (already within +-6) -> 4-bit E2M1 codes, round to
    nearest, ties to even."""
    codes = np.arange(8, dtype=np.uint8)  # 0 .. 7: 0, 0.5, 1, 1.5, 2, 3, 4, 6
    values = decode_e2m1(codes)
    c, neg = _nearest_code(x, codes, values)
    return (c | np.where(neg, 0x8, 0x0)).astype(np.uint8)


def quantize_fp8_1x128(X):
    """X float32 [M, K] (BF16 values) -> (codes uint8 [M, K], scale float32
    [M, K/128])."""
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    assert K % 128 == 0
    Xb = X.reshape(M, K // 128, 128)
    amax = np.abs(Xb).max(axis=2)
    scale = np.where(amax > 0, amax / E4M3_MAX, np.float32(1.0)).astype(np.float32)
    y = (Xb / scale[:, :, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3fn_round(y).reshape(M, K), scale


def nvfp4_global_scale(X) -> np.float32:
    amax = np.float32(np.abs(np.asarray(X, dtype=np.float32)).max()) if np.size(X) else np.float32(0)
    g = np.float32(amax / np.float32(6.0 * 448.0))
    return g if g > 0 else np.float32(1.0)


def quantize_nvfp4(X, g=None):
    """X float32 [M, K] (BF16 values) -> (packed uint8 [M, K/2], scale codes
    uint8 [M, K/16], g float32)."""
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    assert K % 16 == 0
    g = nvfp4_global_scale(X) if g is None else np.float32(g)
    Xb = X.reshape(M, K // 16, 16)
    bamax = np.abs(Xb).max(axis=2)
    s_in = (bamax / (np.float32(6.0) * g)).astype(np.float32)
    s_code = e4m3fn_round(np.minimum(s_in, E4M3_MAX))
    d = (decode_e4m3fn(s_code).astype(np.float32) * g).astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1.0)).astype(np.float32)
    y = np.clip((Xb / safe[:, :, None]).astype(np.float32), -E2M1_MAX, E2M1_MAX)
    q = np.where(d[:, :, None] > 0, e2m1_round(y), np.uint8(0)).reshape(M, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_code, g
