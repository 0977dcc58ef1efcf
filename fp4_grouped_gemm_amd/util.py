"""Host-side helpers for problems held as NumPy dicts (the format of the
seeded workload generators): upload the operands to the current GPU, launch
the library entry point that matches the problem, and read BF16 results
back as float64.  Argument marshalling only, like the rest of the binding."""
from __future__ import annotations

import numpy as np

from . import fp4_gemm, grouped_fp4_gemm, grouped_fp8_gemm

_OPERANDS = ("A", "B", "a_scale", "b_scale", "m_indices")


def to_device(p: dict) -> dict:
    """The problem's operand arrays as contiguous tensors on the current GPU
    (None where the problem has none, e.g. m_indices of a dense problem)."""
    import torch
    return {k: (None if p.get(k) is None else
                torch.from_numpy(np.ascontiguousarray(p[k])).cuda()) for k in _OPERANDS}


def c_to_f64(C) -> np.ndarray:
    """A BF16 tensor (any device) as a float64 NumPy array (exact)."""
    import torch
    bits = C.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def row_ids(p: dict, rows=None):
    """The problem's expert ids with out-of-range values as -1 (the library's
    rule), optionally for a subset of rows; None for a dense problem."""
    m = p.get("m_indices")
    if m is None:
        return None
    m = np.where((m >= 0) & (m < p["G"]), m, -1)
    return m if rows is None else m[rows]


def run(p: dict, d=None, **kw):
    """Launch the entry point for problem p (grouped FP8, dense NVFP4 or
    grouped NVFP4) on its device operands d (uploaded if None); returns C."""
    d = d or to_device(p)
    if p["kind"] == "fp8":
        return grouped_fp8_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"], **kw)
    if p.get("m_indices") is None:
        return fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], p["alpha"], **kw)
    return grouped_fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                            p["alpha"], **kw)
