"""Input quantisers: float arrays -> E4M3FN / E2M1 codes plus block scales.

The recipes follow the problem statement of the block-scaled GEMM:

* FP8: E4M3FN codes (the OCP "FN" variant: bias 7, no infinities, one NaN
  pattern per sign, largest finite 448 -- the gfx950 format named on the
  sglang#27745 page, section "Code analysis 1: FP8 quantisation").  Values are
  clamped to +-448 before encoding, as that page's software encoder does,
  then rounded to nearest, ties to even.  A gets one FP32 scale per row per
  128-wide K block, B one FP32 scale per 128x128 block; each scale is the
  block's amax / 448 (an all-zero block gets scale 1.0).
* NVFP4: E2M1 element codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
  negatives), one E4M3 scale per 16 consecutive K elements and one FP32 global
  scale per tensor.  Reading used: g = amax(tensor) / (6 * 448),
  s = E4M3(amax(block) / (6 g)), q = E2M1(x / (s g)), saturating at +-6, so
  the stored value decodes to q * s * g.  Two codes share a byte, element 2j
  in the low nibble of byte j.

Everything here is vectorised NumPy; nothing is shared with the oracle.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3fn_encode(x) -> np.ndarray:
    """Round float values to E4M3FN codes (RNE, saturating to +-448).

    Works on the FP32 bit pattern: in the normal range the 23-bit FP32
    significand is rounded to 3 bits (half to even, a carry moves into the
    exponent) and the exponent is rebased from bias 127 to bias 7; below
    2**-6 the value is a multiple of the subnormal step 2**-9.  The sign bit
    of the input is kept, so -0.0 and small negatives give code 0x80.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    sign = ((bits >> 31).astype(np.uint8) << 7)
    a = np.minimum(np.abs(x), np.float32(E4M3_MAX))
    ab = a.view(np.uint32)
    rounded = (ab + np.uint32((1 << 19) - 1) + ((ab >> 20) & 1)) >> 20
    normal_code = rounded.astype(np.int64) - ((127 - 7) << 3)
    sub_code = np.rint(a * np.float32(512.0)).astype(np.int64)
    code = np.where(a >= np.float32(2.0 ** -6), normal_code, sub_code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3fn_values() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (NaN codes give NaN); used by
    the NVFP4 quantiser to divide by the rounded block scale."""
    c = np.arange(256)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 7
    mag = np.where(E == 0, M * 2.0 ** -9, (8 + M) * np.ldexp(1.0, E - 10))
    v = s * mag
    v[(c & 0x7F) == 0x7F] = np.nan
    return v


def e2m1_encode(x) -> np.ndarray:
    """Round float values to 4-bit E2M1 codes (RNE, saturating to +-6).

    For |x| >= 1 the FP32 significand is rounded to 1 bit (half to even) and
    the exponent rebased from bias 127 to bias 1; below 1 the value is a
    multiple of the subnormal step 0.5.
    """
    x = np.asarray(x, dtype=np.float32)
    sign = ((x.view(np.uint32) >> 31).astype(np.uint8) << 3)
    a = np.minimum(np.abs(x), np.float32(E2M1_MAX))
    ab = a.view(np.uint32)
    rounded = (ab + np.uint32((1 << 21) - 1) + ((ab >> 22) & 1)) >> 22
    normal_code = rounded.astype(np.int64) - ((127 - 1) << 1)
    sub_code = np.rint(a * np.float32(2.0)).astype(np.int64)
    code = np.where(a >= np.float32(1.0), normal_code, sub_code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def _block_scale(amax: np.ndarray, fmax: float) -> np.ndarray:
    s = (amax / fmax).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _row_chunks(fn, X: np.ndarray, align: int):
    """Apply ``fn`` to row chunks of X (chunk sizes multiples of ``align``) on a
    thread pool and concatenate each of its outputs along axis 0.  NumPy
    releases the GIL inside the element-wise kernels, so this scales with
    cores; the result is identical to ``fn(X)``."""
    R = X.shape[0]
    n = _workers()
    step = max(align, -(-R // (4 * n)) // align * align)
    if R <= step:
        return fn(X)
    parts = [X[i:i + step] for i in range(0, R, step)]
    with ThreadPoolExecutor(n) as ex:
        outs = list(ex.map(fn, parts))
    if isinstance(outs[0], tuple):
        return tuple(np.concatenate([o[j] for o in outs]) for j in range(len(outs[0])))
    return np.concatenate(outs)


def quantize_fp8_rows(X: np.ndarray):
    """X[R, K] -> (codes uint8 [R, K], a_scale float32 [R, K/128])."""
    return _row_chunks(_quantize_fp8_rows, X, 1)


def _quantize_fp8_rows(X: np.ndarray):
    R, K = X.shape
    assert K % 128 == 0
    Xb = X.reshape(R, K // 128, 128)
    scale = _block_scale(np.abs(Xb).max(axis=2), E4M3_MAX)
    codes = e4m3fn_encode(Xb / scale[:, :, None])
    return codes.reshape(R, K), scale


def quantize_fp8_blocks(X: np.ndarray):
    """X[N, K] (one expert) -> (codes uint8 [N, K], scale float32 [N/128, K/128])."""
    return _row_chunks(_quantize_fp8_blocks, X, 128)


def _quantize_fp8_blocks(X: np.ndarray):
    N, K = X.shape
    assert N % 128 == 0 and K % 128 == 0
    Xb = X.reshape(N // 128, 128, K // 128, 128)
    scale = _block_scale(np.abs(Xb).max(axis=(1, 3)), E4M3_MAX)
    codes = e4m3fn_encode(Xb / scale[:, None, :, None])
    return codes.reshape(N, K), scale


def nvfp4_global_scale(amax: float) -> np.float32:
    g = np.float32(amax / (E2M1_MAX * E4M3_MAX))
    return g if g > 0 else np.float32(1.0)


def quantize_nvfp4(X: np.ndarray, g: np.float32 | None = None):
    """X[R, K] -> (packed uint8 [R, K/2], scale codes uint8 [R, K/16], g float32).

    ``g`` is computed from X's amax unless given (a grouped B shares one g
    over all experts).
    """
    if g is None:
        g = nvfp4_global_scale(float(np.abs(X).max()))
    g32 = np.float32(g)
    packed, s_code = _row_chunks(lambda Xc: _quantize_nvfp4(Xc, g32), X, 1)
    return packed, s_code, g32


def _quantize_nvfp4(X: np.ndarray, g32: np.float32):
    R, K = X.shape
    assert K % 16 == 0
    Xb = X.reshape(R, K // 16, 16)
    bamax = np.abs(Xb).max(axis=2)
    s_code = e4m3fn_encode(bamax / (np.float32(E2M1_MAX) * g32))
    s_val = e4m3fn_values().astype(np.float32)[s_code]
    denom = s_val * g32
    safe = np.where(denom > 0, denom, np.float32(1.0)).astype(np.float32)
    q = e2m1_encode(np.where(denom[:, :, None] > 0, Xb / safe[:, :, None], np.float32(0.0)))
    q = q.reshape(R, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_code.astype(np.uint8)
