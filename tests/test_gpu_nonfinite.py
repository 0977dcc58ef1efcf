"""Non-finite values on the GPU, through the C ABI.

* E4M3FN NaN scale codes (0x7F / 0xFF) in the NVFP4 GEMMs: every output a
  NaN scale reaches is NaN, as in the oracle (which decodes the scale codes
  from the format definition, NaN included); all other outputs match it.
* Bytes that the method never multiplies -- activation rows routed to -1,
  the memory right after A -- may hold Inf / NaN: W4A16 with K an odd
  multiple of 128 (a half-full last K group) and the grouped FP8 GEMM with
  padding rows of NaN codes still give finite, oracle-matching valid rows
  and exactly zero padding rows.
"""
import numpy as np
import pytest

import oracle
import fp4_grouped_gemm_amd as fgg
from tests.gpu_util import c_bits, c_to_f64, log, to_dev
from workloads import fp8_problem, nvfp4_problem, runs_to_indices, w4a16_problem

pytestmark = pytest.mark.gpu

BF16_NAN, BF16_INF = 0x7FC0, 0x7F80


def _nan_mask_check(out, ref, what):
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan_ref), f"{what}: NaN positions differ"
    rows = ~nan_ref.any(axis=1)
    cols = ~nan_ref.any(axis=0)
    res = oracle.check_tolerance(out[np.ix_(rows, cols)], ref[np.ix_(rows, cols)])
    assert res["ok"], f"{what}: {res}"


@pytest.mark.parametrize("grouped", [False, True])
def test_nvfp4_nan_scale_codes_propagate(grouped):
    rng = np.random.default_rng(21)
    if grouped:
        ids = runs_to_indices([70, 0, 90, 40])
        p = nvfp4_problem(ids, ids.size, 256, 384, 4, rng)
    else:
        p = nvfp4_problem(None, 200, 256, 384, 1, rng)
    sa, sb = p["a_scale"].copy(), p["b_scale"].copy()
    sa[17, 5] = 0x7F   # +NaN code: row 17
    sa[150, 23] = 0xFF  # -NaN code: row 150
    if grouped:
        sb[2, 33, 0] = 0x7F  # expert 2, column 33
    else:
        sb[33, 0] = 0x7F
    p = dict(p, a_scale=sa, b_scale=sb)
    d = to_dev(p)
    log(f"nvfp4 NaN scale codes grouped={grouped}")
    if grouped:
        C = fgg.grouped_fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                                 p["alpha"])
        with np.errstate(invalid="ignore"):
            ref = oracle.grouped_fp4_gemm(p["A"], p["B"], sa, sb, p["m_indices"], p["alpha"])
    else:
        C = fgg.fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], p["alpha"])
        with np.errstate(invalid="ignore"):
            ref = oracle.fp4_gemm(p["A"], p["B"], sa, sb, p["alpha"])
    assert np.isnan(ref).any()
    _nan_mask_check(c_to_f64(C), ref, f"grouped={grouped}")


def test_w4a16_odd_k_ignores_nonfinite_neighbours():
    """K = 640 = 5 x 128: the last 256-wide K group is half full.  Rows
    routed to -1 hold Inf / NaN, and so does a guard row right after A; the
    valid rows must match the oracle and stay finite."""
    import torch
    ids = np.array([0, -1, 1, -1, 0, 2, 2, -1, 1], np.int32)
    p = w4a16_problem(ids, 256, 640, 3, np.random.default_rng(22))
    M, K = p["M"], p["K"]
    bits = np.empty((M + 1, K), np.uint16)
    bits[:M] = p["A_bits"]
    for i in np.nonzero(ids < 0)[0]:
        bits[i] = BF16_INF if i % 2 else BF16_NAN
    bits[M] = BF16_NAN  # guard row right after A
    buf = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    A = buf[:M]
    d = dict(B=torch.from_numpy(p["B"]).cuda(), b_scale=torch.from_numpy(p["b_scale"]).cuda(),
             m_indices=torch.from_numpy(ids).cuda())
    log("w4a16 K=640 with non-finite neighbours")
    C = fgg.grouped_w4a16_gemm(A, d["B"], d["b_scale"], d["m_indices"], p["b_global"])
    ref = oracle.grouped_w4a16_gemm(p["A"], p["B"], p["b_scale"], ids, p["b_global"])
    res = oracle.check_tolerance(c_to_f64(C), ref, ids)
    assert res["ok"], res


def test_fp8_nan_padding_rows_stay_out():
    """Padding rows (m_indices = -1) filled with E4M3 NaN codes share 8-row
    load groups and MFMA row blocks with valid rows; every valid row must
    match the oracle and every padding row be exactly zero."""
    ids = runs_to_indices([37, 60, 3], pad_to=16)
    ids = np.concatenate([ids, np.full(11, -1, np.int32)])
    p = fp8_problem(ids, 256, 512, 3, np.random.default_rng(23))
    A = p["A"].copy()
    A[ids < 0] = 0x7F
    p = dict(p, A=A)
    d = to_dev(p)
    for tile in range(fgg.num_tiles(fgg.FP8)):
        log(f"fp8 NaN padding rows tile={tile}")
        C = fgg.grouped_fp8_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                                 tile_id=tile)
        ref = oracle.grouped_fp8_gemm(A, p["B"], p["a_scale"], p["b_scale"], ids)
        res = oracle.check_tolerance(c_to_f64(C), ref, ids)
        assert res["ok"], (tile, res)
        assert np.all(c_bits(C)[ids < 0] == 0)


def test_nvfp4_every_scale_code_through_the_kernel():
    """All 256 E4M3FN codes as A block scales, one per row: A and B values
    all 1.0 (E2M1 0x2), B scales 1.0 (0x38), alpha 1, K = 128 with only the
    first 16-element block of each A row scaled (the others code 0), so
    C[r, n] = 16 * value(code r) exactly -- BF16-exact for every finite
    code, NaN for 0x7F and 0xFF.  Checked bitwise against the oracle's
    decode of the format, on every tile config."""
    M, N, K = 256, 128, 128
    A = np.full((M, K // 2), 0x22, np.uint8)
    B = np.full((N, K // 2), 0x22, np.uint8)
    sa = np.zeros((M, K // 16), np.uint8)
    sa[:, 0] = np.arange(256, dtype=np.uint8)
    sb = np.full((N, K // 16), 0x38, np.uint8)
    with np.errstate(invalid="ignore"):
        ref = oracle.fp4_gemm(A, B, sa, sb, 1.0)
    nan = np.isnan(ref)
    assert nan.any(axis=1).sum() == 2
    want = oracle.bf16_rne_bits(np.where(nan, 0.0, ref))
    p = dict(kind="nvfp4", A=A, B=B, a_scale=sa, b_scale=sb, m_indices=None, alpha=1.0,
             M=M, N=N, K=K, G=1)
    d = to_dev(p)
    for tile in range(fgg.num_tiles(fgg.FP4)):
        log(f"nvfp4 all scale codes tile={tile}")
        C = fgg.fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], 1.0, tile_id=tile)
        got = c_bits(C)
        assert np.array_equal(np.isnan(c_to_f64(C)), nan), tile
        assert np.array_equal(got[~nan], want[~nan]), tile
