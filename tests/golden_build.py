"""Builds problem arrays from the hand-computed worked examples in
``tests/golden/worked_examples.json`` (see that file's "about" note for the
sources).  Used by the oracle pins and by the GPU parity tests."""
from __future__ import annotations

import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load_examples():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["examples"]


def build(ex: dict) -> dict:
    kind, M, N, K, G = ex["kind"], ex["M"], ex["N"], ex["K"], ex["G"]
    fp4 = kind == "nvfp4"
    kdiv = 16 if fp4 else 128
    # element codes, unpacked
    A = np.full((M, K), ex["A"]["fill"], np.uint8)
    for i, code in ex["A"].get("set_rows", []):
        A[i, :] = code
    for i, k, code in ex["A"].get("set", []):
        A[i, k] = code
    B = np.full((G, N, K), ex["B"]["fill"], np.uint8)
    for g, code in ex["B"].get("expert_fill", []):
        B[g] = code
    for g, n, k, code in ex["B"].get("set", []):
        B[g, n, k] = code
    sdt = np.uint8 if fp4 else np.float32
    a_scale = np.full((M, K // kdiv), ex["a_scale"]["fill"], sdt)
    for i, kb, v in ex["a_scale"].get("set", []):
        a_scale[i, kb] = v
    bshape = (G, N, K // 16) if fp4 else (G, N // 128, K // 128)
    b_scale = np.full(bshape, ex["b_scale"]["fill"], sdt)
    for g, nb, kb, v in ex["b_scale"].get("set", []):
        b_scale[g, nb, kb] = v
    for blk, v in ex["b_scale"].get("set_cols", []):
        b_scale[:, :, blk] = v
    m_idx = ex["m_indices"]
    d = dict(kind=kind, M=M, N=N, K=K, G=G, a_scale=a_scale, b_scale=b_scale,
             m_indices=None if m_idx is None else np.array(m_idx, np.int32))
    if fp4:
        A = (A[:, 0::2] & 0xF) | ((A[:, 1::2] & 0xF) << 4)
        B = (B[..., 0::2] & 0xF) | ((B[..., 1::2] & 0xF) << 4)
        d["alpha"] = np.float32(ex["alpha"])
        if m_idx is None:
            B, d["b_scale"] = B[0], b_scale[0]
    d["A"], d["B"] = A.astype(np.uint8), B.astype(np.uint8)
    exp = np.full((M, N), np.nan)
    bits = np.zeros((M, N), np.uint16)
    for r, c0, c1, v in ex["expected"]:
        exp[r, c0:c1] = v
    for r, c0, c1, v in ex["expected_bf16"]:
        bits[r, c0:c1] = v
    assert not np.isnan(exp).any(), ex["name"]
    d["expected"], d["expected_bf16"] = exp, bits
    return d
