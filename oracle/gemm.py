"""Float64 reference for block-scaled FP8 / NVFP4 (grouped) GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources of the definitions:
  * flashinfer#7877 page ("cake_grouped_fp8_gemm" window-segment program),
    sections "Intro" and "Code analysis 1": FP8 E4M3 inputs, BF16 output,
    rows grouped by m_indices, FP32 per-128 block scales; the kernel takes
    A, B, C, a_scale, b_scale, m_indices, M, N, K, G, and A's descriptor is a
    row-major [M, K] byte matrix with K a multiple of 128.
  * onnxruntime#29824 page, "Code analysis 1": NVFP4 W4A4 grouped GEMM for
    MoE prefill; flashinfer#3948 page: dense NVFP4 mm_fp4.
Readings where the pages are silent: a_scale is [M, K/128] row-major (one
scale per row per 128-K block), b_scale is [G, N/128, K/128] row-major (one per
128x128 block of B[g]), B is [G, N, K] with K contiguous, C is [M, N] row
major; m_indices is int32[M] holding an expert id in [0, G) or -1 for a
padding row whose output is exactly zero.  NVFP4 scales are row-major
[rows, K/16] E4M3 codes and the two global scales enter only as their product
alpha = gA * gB.

Every function accepts ``rows`` (an index array) to compute only those rows of
C, so large problems can be checked on a sample of outputs.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e2m1, decode_e4m3fn, unpack_e2m1

_E4M3_LUT = decode_e4m3fn(np.arange(256, dtype=np.uint8))
_E2M1_LUT = decode_e2m1(np.arange(16, dtype=np.uint8))


def _rows_arg(rows, M):
    if rows is None:
        return np.arange(M)
    rows = np.asarray(rows, dtype=np.int64)
    assert rows.ndim == 1 and (rows.size == 0 or (rows.min() >= 0 and rows.max() < M))
    return rows


def grouped_fp8_gemm(A, B, a_scale, b_scale, m_indices, rows=None) -> np.ndarray:
    """C (float64, [len(rows), N]) of the grouped FP8 block-scaled GEMM.

    For each expert g and each 128-wide K block kb, the block product of the
    decoded E4M3 values is formed in float64 -- exact, because every E4M3
    value is an integer times 2^-9, so each term is an integer times 2^-18
    and a 128-term sum stays far below 2^53 of them -- then multiplied by
    a_scale[i, kb] * b_scale[g, n // 128, kb] and summed over kb in float64.
    Parity: pinned (exhaustive decode, exact rational brute force, worked
    examples, invariants).
    """
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    a_scale = np.asarray(a_scale, np.float32)
    b_scale = np.asarray(b_scale, np.float32)
    m_indices = np.asarray(m_indices, np.int32)
    M, K = A.shape
    G, N, Kb = B.shape
    assert Kb == K and K % 128 == 0 and N % 128 == 0
    assert a_scale.shape == (M, K // 128)
    assert b_scale.shape == (G, N // 128, K // 128)
    assert m_indices.shape == (M,)
    assert np.all((m_indices >= -1) & (m_indices < G)), "expert ids must lie in [-1, G)"
    rows = _rows_arg(rows, M)
    C = np.zeros((rows.size, N), dtype=np.float64)
    ids = m_indices[rows]
    for g in range(G):
        sel = np.nonzero(ids == g)[0]
        if sel.size == 0:
            continue
        r = rows[sel]
        Ad = _E4M3_LUT[A[r]]  # [R, K]
        Bd = _E4M3_LUT[B[g]]  # [N, K]
        acc = np.zeros((r.size, N), dtype=np.float64)
        for kb in range(K // 128):
            ks = slice(kb * 128, (kb + 1) * 128)
            P = Ad[:, ks] @ Bd[:, ks].T  # exact block partial sums
            sa = a_scale[r, kb].astype(np.float64)
            sb = np.repeat(b_scale[g, :, kb].astype(np.float64), 128)
            acc += (sa[:, None] * sb[None, :]) * P
        C[sel] = acc
    return C


def _nvfp4_dequant(packed, scale_codes) -> np.ndarray:
    """Packed E2M1 [R, K/2] and E4M3 block scales [R, K/16] -> q * s in
    float64 (exact: at most 6 significant bits)."""
    q = _E2M1_LUT[unpack_e2m1(packed)]
    s = _E4M3_LUT[np.asarray(scale_codes, np.uint8)]
    R, K = q.shape
    assert s.shape == (R, K // 16)
    return (q.reshape(R, K // 16, 16) * s[:, :, None]).reshape(R, K)


def fp4_gemm(A, B, a_scale, b_scale, alpha, rows=None) -> np.ndarray:
    """C (float64, [len(rows), N]) of the dense NVFP4 GEMM.

    Scales are folded into the operands exactly (E2M1 x E4M3 needs at most
    6 significant bits), one float64 GEMM follows, then the product is
    multiplied by alpha = gA * gB.  This equals the per-16-block form
    alpha * sum_kb sA sB sum_k qA qB in exact arithmetic.
    Parity: pinned (exact integer brute force, worked examples, invariants).
    """
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    M, K2 = A.shape
    N, K2b = B.shape
    assert K2 == K2b
    rows = _rows_arg(rows, M)
    Ad = _nvfp4_dequant(A[rows], np.asarray(a_scale)[rows])
    Bd = _nvfp4_dequant(B, b_scale)
    return float(np.float32(alpha)) * (Ad @ Bd.T)


def grouped_fp4_gemm(A, B, a_scale, b_scale, m_indices, alpha, rows=None) -> np.ndarray:
    """C (float64, [len(rows), N]) of the grouped NVFP4 GEMM: row i uses
    B[g], b_scale[g] with g = m_indices[i]; rows with g = -1 are zero.
    ``alpha`` is one float (one global scale for every expert's B) or a
    sequence of G floats, alpha[g] = gA * gB[g] (a global scale per expert:
    the per-group scaling of the cutlass#3124 page's grouped block-scaled
    GEMM); either way expert g's rows are multiplied by its alpha.
    Parity: pinned (G = 1 equals the dense form; brute force with distinct
    per-expert alphas; invariants)."""
    A = np.asarray(A, np.uint8)
    B = np.asarray(B, np.uint8)
    m_indices = np.asarray(m_indices, np.int32)
    M, K2 = A.shape
    G, N, K2b = B.shape
    assert K2 == K2b and m_indices.shape == (M,)
    assert np.all((m_indices >= -1) & (m_indices < G)), "expert ids must lie in [-1, G)"
    alphas = np.broadcast_to(np.asarray(alpha, np.float32), (G,))
    rows = _rows_arg(rows, M)
    ids = m_indices[rows]
    C = np.zeros((rows.size, N), dtype=np.float64)
    for g in range(G):
        sel = np.nonzero(ids == g)[0]
        if sel.size == 0:
            continue
        r = rows[sel]
        C[sel] = fp4_gemm(A[r], B[g], np.asarray(a_scale)[r], np.asarray(b_scale)[g], alphas[g])
    return C


def grouped_w4a16_gemm(A, B, b_scale, m_indices, b_global, rows=None) -> np.ndarray:
    """C (float64, [len(rows), N]) of the grouped W4A16 GEMM: 16-bit
    activations times NVFP4 weights (the onnxruntime#29824 page, "Code
    analysis 1": FP4 weights with 16-bit activations, dequantised, on the
    decode / small-M path).  A [M, K] holds BF16 values (as float32 or
    float64), B [G, N, K/2] packed E2M1 with E4M3 block scales b_scale [G, N,
    K/16] and one FP32 global scale b_global for all experts:
      C[i, n] = b_global * sum_k A[i, k] * qB[g, n, k] * sB[g, n, k/16],
    g = m_indices[i]; rows with g = -1 are zero.  B is dequantised exactly
    (at most 6 significant bits) and multiplied in float64.
    Parity: pinned (inputs that are exactly NVFP4 reproduce the W4A4 form;
    exact rational brute force; padding rows)."""
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.uint8)
    m_indices = np.asarray(m_indices, np.int32)
    M, K = A.shape
    G, N, K2 = B.shape
    assert 2 * K2 == K and m_indices.shape == (M,)
    assert np.all((m_indices >= -1) & (m_indices < G)), "expert ids must lie in [-1, G)"
    rows = _rows_arg(rows, M)
    ids = m_indices[rows]
    gb = float(np.float32(b_global))
    C = np.zeros((rows.size, N), dtype=np.float64)
    for g in range(G):
        sel = np.nonzero(ids == g)[0]
        if sel.size == 0:
            continue
        Bd = _nvfp4_dequant(B[g], np.asarray(b_scale)[g])
        C[sel] = gb * (A[rows[sel]] @ Bd.T)
    return C


def fp4_gemm_problems(problems) -> list:
    """A batch of independent dense NVFP4 GEMMs of different shapes in one
    call (cutlass#3124 page, "Intro": one launch runs several GEMMs whose M,
    N and K differ).  ``problems`` is a sequence of dicts with A [M, K/2], B
    [N, K/2], a_scale [M, K/16], b_scale [N, K/16] and alpha; the result is
    the list of their C (float64 [M, N]), each exactly fp4_gemm of its
    problem.  Parity: pinned (row and column slices of one problem tile that
    problem's result; exact brute force)."""
    return [fp4_gemm(q["A"], q["B"], q["a_scale"], q["b_scale"], q["alpha"]) for q in problems]


def rms_nonpadding(ref, ids=None) -> float:
    """Root mean square of the reference over non-padding rows."""
    ref = np.asarray(ref, np.float64)
    if ids is not None:
        ref = ref[np.asarray(ids) >= 0]
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def check_tolerance(out, ref, ids=None, rtol=1e-2, rms_frac=1e-3) -> dict:
    """Acceptance rule for a kernel output against this oracle.

    Every non-padding element must satisfy |C - ref| <= rtol * |ref| +
    rms_frac * rms(ref), rms over the non-padding elements given; padding rows
    (ids == -1) must be exactly zero.  Returns a summary with ``ok``.
    """
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape
    pad = np.zeros(out.shape[0], bool) if ids is None else (np.asarray(ids) < 0)
    rms = rms_nonpadding(ref, None if ids is None else ids)
    real = ~pad
    err = np.abs(out[real] - ref[real])
    bound = rtol * np.abs(ref[real]) + rms_frac * rms
    bad = err > bound
    pad_bad = int(np.count_nonzero(out[pad] != 0.0)) if pad.any() else 0
    nan_bad = int(np.count_nonzero(~np.isfinite(out[real])))
    worst = float(np.max(err / np.where(bound > 0, bound, 1.0))) if err.size else 0.0
    return dict(ok=(not bad.any()) and pad_bad == 0 and nan_bad == 0,
                n_bad=int(np.count_nonzero(bad)), n_pad_nonzero=pad_bad, n_nonfinite=nan_bad,
                worst_ratio=worst, rms=rms, n=int(err.size))
