"""GPU parity of fp4_gemm / grouped_fp4_gemm against the float64 oracle
(through the C ABI)."""
import numpy as np
import pytest

import oracle
from tests.golden_build import build, load_examples
from tests.gpu_util import assert_parity, c_bits, c_to_f64, log, ref, run, sample_rows, to_dev
from workloads import make, nvfp4_problem, runs_to_indices

pytestmark = pytest.mark.gpu

FP4_TILES = [0, 1, 2, 3]


@pytest.mark.parametrize("ex", [e for e in load_examples() if e["kind"] == "nvfp4"],
                         ids=lambda e: e["name"])
def test_worked_examples_bitwise(ex):
    d = build(ex)
    for tile in FP4_TILES:
        log(f"worked example {ex['name']} tile {tile}")
        assert np.array_equal(c_bits(run(d, tile_id=tile)), d["expected_bf16"]), (ex["name"], tile)


def test_every_code_and_scale_pair_exact():
    """All 16 E2M1 codes x all 254 non-NaN E4M3 scale codes: with B the
    identity (one nonzero product per output) C[i, n] is the dequantised
    A[i, n] itself, exact in BF16, so it must match bitwise."""
    scales = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    nb = scales.size  # one 16-element block per scale code, holding codes 0..15
    K = 128
    M = -(-nb // (K // 16))
    codes = np.zeros((M, K), np.uint8)
    sa = np.full((M, K // 16), 0x38, np.uint8)
    for b, s in enumerate(scales):
        i, blk = divmod(b, K // 16)
        codes[i, blk * 16:(blk + 1) * 16] = np.arange(16)
        sa[i, blk] = s
    A = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    eye = np.where(np.eye(K, dtype=bool), 0x2, 0x0).astype(np.uint8)  # E2M1 1.0 on the diagonal
    B = (eye[:, 0::2] | (eye[:, 1::2] << 4)).astype(np.uint8)
    sb = np.full((K, K // 16), 0x38, np.uint8)
    p = dict(kind="nvfp4", M=M, N=K, K=K, G=1, A=A, B=B, a_scale=sa, b_scale=sb,
             alpha=np.float32(1.0), m_indices=None)
    want = oracle.bf16_rne_bits(ref(p))
    for tile in FP4_TILES:
        log(f"exhaustive dequant tile {tile}")
        assert np.array_equal(c_bits(run(p, tile_id=tile)), want), tile


def _dense(M, N, K, seed=0):
    return nvfp4_problem(None, M, N, K, 1, np.random.default_rng(seed))


def _grouped(ids, N=256, K=512, G=None, seed=0):
    ids = np.asarray(ids, np.int32)
    G = G or max(1, int(ids.max()) + 1)
    return nvfp4_problem(ids, ids.size, N, K, G, np.random.default_rng(seed))


CASES = {
    "dense_small": lambda: _dense(200, 256, 512),
    "dense_M1": lambda: _dense(1, 128, 128),
    "dense_ragged": lambda: _dense(333, 384, 1152, seed=3),
    "grouped_runs": lambda: _grouped(runs_to_indices([70, 0, 130, 57], pad_to=8)),
    "grouped_all_padding": lambda: _grouped([-1] * 130, G=2),
    "grouped_unsorted": lambda: _grouped(np.random.default_rng(5).integers(-1, 4, 301), G=4),
    "grouped_out_of_range": lambda: _grouped([0, 9, -3, 1] * 50, G=2),
    "grouped_run_of_one": lambda: _grouped([0] * 60 + [1] + [2] * 90, G=3),
    # more experts than tile rows (split mode: item r runs expert r)
    "grouped_more_experts_than_rows": lambda: _grouped(
        np.random.default_rng(12).integers(-1, 300, 400), G=300),
    # K loops of 6, 10, 14 and 12 steps of 64: every exit position of the
    # eight-step unrolled loop and of the four-step scale groups
    "dense_k384": lambda: _dense(130, 256, 384, seed=6),
    "dense_k640": lambda: _dense(77, 128, 640, seed=7),
    "grouped_k896": lambda: _grouped(runs_to_indices([40, 90, 0, 33]), N=256, K=896, seed=8),
    "grouped_k768": lambda: _grouped(runs_to_indices([129, 127, 3]), N=384, K=768, seed=9),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("tile", FP4_TILES)
def test_cases(case, tile):
    p = CASES[case]()
    log(f"fp4 {case} tile {tile} M={p['M']} N={p['N']} K={p['K']} G={p['G']}")
    assert_parity(p, run(p, tile_id=tile), what=f"{case}/tile{tile}")


def test_grouped_single_expert_equals_dense_bitwise():
    p = _grouped([0] * 300, N=256, K=512, G=1)
    d = to_dev(p)
    log("grouped G=1 vs dense")
    import fp4_grouped_gemm_amd as fgg
    Cg = fgg.grouped_fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"], p["alpha"])
    Cd = fgg.fp4_gemm(d["A"], d["B"][0], d["a_scale"], d["b_scale"][0], p["alpha"])
    assert np.array_equal(c_bits(Cg), c_bits(Cd))


@pytest.mark.parametrize("case", ["grouped_runs", "grouped_unsorted", "grouped_out_of_range",
                                  "grouped_run_of_one", "grouped_all_padding", "grouped_k896",
                                  "grouped_more_experts_than_rows"])
def test_run_split_modes_agree_bitwise(case):
    """Split mode (each expert pass of a window its own workgroup) against
    one workgroup per window: same bits, and within the oracle's tolerance."""
    p = CASES[case]()
    d = to_dev(p)
    for tile in FP4_TILES:
        log(f"fp4 run split {case} tile {tile}")
        split = c_bits(run(p, d, tile_id=tile, run_split=1)).copy()
        C = run(p, d, tile_id=tile, run_split=-1)
        assert np.array_equal(split, c_bits(C)), (case, tile)
        assert_parity(p, C, what=f"split {case}/tile{tile}")
    log(f"fp4 run split {case} capped grid")
    assert_parity(p, run(p, d, run_split=1, max_workgroups=3), what=f"split {case} capped")


@pytest.mark.parametrize("max_wg", [1, 5])
def test_persistent_loop(max_wg):
    p = _grouped(runs_to_indices([100, 300, 11, 200]), N=384, K=256)
    for tile in FP4_TILES:
        log(f"fp4 persistent max_wg={max_wg} tile {tile}")
        assert_parity(p, run(p, tile_id=tile, max_workgroups=max_wg), what=f"{max_wg}/{tile}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c4_dense_nvfp4", "c5_moe_nvfp4"])
def test_full_size_sampled(name):
    p = make(name)
    d = to_dev(p)
    rows = sample_rows(p, 160)
    log(f"{name} full size, ranker's tile")
    C = run(p, d)
    assert_parity(p, C, rows=rows, what=name)
    assert np.all(np.isfinite(c_to_f64(C)))
    # Every tile shape accumulates each output over the same K steps with the
    # same MFMA, so all of them give the same bits: compared on every element,
    # and each against the oracle on a sample of rows.
    bits = c_bits(C).copy()
    del C
    for tile in FP4_TILES:
        log(f"{name} full size tile {tile}")
        Ct = run(p, d, tile_id=tile)
        assert_parity(p, Ct, rows=rows[::4], what=f"{name}/tile{tile}")
        assert np.array_equal(c_bits(Ct), bits), (name, tile)
        del Ct
