"""Helpers shared by the GPU tests: upload a workload, run the library, read
C back as float64, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import fp4_grouped_gemm_amd as fgg  # noqa: F401
import oracle
from fp4_grouped_gemm_amd.util import c_to_f64, row_ids, run  # noqa: F401
from fp4_grouped_gemm_amd.util import to_device as to_dev  # noqa: F401


def log(msg: str):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def c_bits(C) -> np.ndarray:
    import torch
    return C.view(torch.int16).cpu().numpy().view(np.uint16)


def ref(p: dict, rows=None, ids=None) -> np.ndarray:
    """Oracle output; out-of-range expert ids act as -1 (the library's rule)."""
    m = p.get("m_indices")
    if m is not None:
        m = np.where((m >= 0) & (m < p["G"]), m, -1).astype(np.int32) if ids is None else ids
    if p["kind"] == "fp8":
        return oracle.grouped_fp8_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], m, rows=rows)
    if m is None:
        return oracle.fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], p["alpha"], rows=rows)
    return oracle.grouped_fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], m, p["alpha"],
                                   rows=rows)


def assert_parity(p: dict, C, rows=None, what=""):
    out = c_to_f64(C)
    if rows is not None:
        out = out[rows]
    r = ref(p, rows=rows)
    res = oracle.check_tolerance(out, r, row_ids(p, rows))
    assert res["ok"], f"{what}: {res}"
    return res


def sample_rows(p: dict, n: int, seed: int = 0) -> np.ndarray:
    """Rows to check at full size: the first and last row of every expert
    run, the rows around every run boundary and window edge, and a seeded
    random sample."""
    M = p["M"]
    rng = np.random.default_rng(seed)
    picks = {0, M - 1}
    m = p.get("m_indices")
    if m is not None:
        b = np.nonzero(np.diff(m) != 0)[0]
        for i in b:
            picks.update({int(i), int(i) + 1})
    for w in range(0, M, 128):
        picks.update({w, min(M - 1, w + 127)})
    picks = sorted(x for x in picks if 0 <= x < M)
    extra = rng.choice(M, size=min(M, max(0, n - len(picks))), replace=False)
    return np.unique(np.concatenate([np.array(picks, np.int64), extra.astype(np.int64)]))
