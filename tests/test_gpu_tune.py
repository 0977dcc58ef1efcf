"""Bounded autotuning through the C ABI: the *_tune calls time the ranker's
top-k tile configs on the caller's inputs, record the fastest for the shape,
and later default calls launch it (flashinfer#3948 page, "Code analysis 1":
profile only the heuristic's top candidates)."""
import numpy as np
import pytest

import fp4_grouped_gemm_amd as fgg
from tests.gpu_util import assert_parity, c_bits, log, run, to_dev
from workloads import fp8_problem, make, nvfp4_problem, runs_to_indices

pytestmark = pytest.mark.gpu


def _tune(p, d, **kw):
    if p["kind"] == "fp8":
        return fgg.grouped_fp8_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"],
                                         d["m_indices"], **kw)
    if p.get("m_indices") is None:
        return fgg.fp4_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"], p["alpha"], **kw)
    return fgg.grouped_fp4_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                                     p["alpha"], **kw)


CASES = {
    "fp8_m777_g8": lambda: make("p2_m777_g8"),
    "fp4_dense": lambda: nvfp4_problem(None, 300, 512, 512, 1, np.random.default_rng(2)),
    "fp4_grouped": lambda: nvfp4_problem(runs_to_indices([90, 0, 170, 40]), 300, 256, 384, 4,
                                         np.random.default_rng(3)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_tune_records_fastest_and_default_calls_use_it(case):
    p = CASES[case]()
    d = to_dev(p)
    kind = fgg.FP8 if p["kind"] == "fp8" else fgg.FP4
    M, N, K, G = p["M"], p["N"], p["K"], p["G"]
    fgg.tune_clear()
    assert fgg.tuned_tile(kind, M, N, K, G) == -1
    log(f"tune {case}")
    C, rep = _tune(p, d, top_k=4, reps=3)
    ranked = [t["id"] for t in fgg.rank_tiles(kind, M, N, K, G,
                                              num_cus=fgg.device_info()["num_cus"])]
    assert rep["tile_id"] == ranked[:len(rep["tile_id"])] and len(rep["tile_id"]) == min(4, len(ranked))
    assert all(t > 0 for t in rep["ms"])
    assert rep["best"] == int(np.argmin(rep["ms"])) and rep["chosen"] == rep["tile_id"][rep["best"]]
    assert fgg.tuned_tile(kind, M, N, K, G) == rep["chosen"]
    assert_parity(p, C, what=f"tune output {case}")
    # a default call now launches the recorded config: same bits as asking for it
    default = c_bits(run(p, d)).copy()
    assert np.array_equal(default, c_bits(run(p, d, tile_id=rep["chosen"])))
    fgg.tune_clear()
    assert fgg.tuned_tile(kind, M, N, K, G) == -1


def test_tune_top1_is_the_heuristic_and_bad_arguments_raise():
    p = make("c1_tiny_fp8")
    d = to_dev(p)
    fgg.tune_clear()
    log("tune top_k=1")
    _, rep = _tune(p, d, top_k=1, reps=1)
    top = fgg.rank_tiles(fgg.FP8, p["M"], p["N"], p["K"], p["G"],
                         num_cus=fgg.device_info()["num_cus"])[0]["id"]
    assert rep["tile_id"] == [top] and rep["chosen"] == top
    with pytest.raises(ValueError, match="top_k"):
        _tune(p, d, top_k=0, reps=1)
    with pytest.raises(ValueError, match="reps"):
        _tune(p, d, top_k=2, reps=0)
    fgg.tune_clear()


def test_run_align_changes_only_the_tile():
    """Runs padded to 128 rows (the MoE alignment step): with run_align=128
    the ranker picks a 128-row tile here (no two-expert windows) where it
    otherwise picks a wider one.  The default call with the promise launches
    exactly that tile (bitwise equal to asking for it) and matches the
    oracle; so does the call without the promise."""
    counts = [128 * k for k in (5, 3, 9, 1, 6, 4, 2, 2)]
    p = fp8_problem(runs_to_indices(counts), 1024, 256, 8, np.random.default_rng(11))
    M, N, K, G = p["M"], p["N"], p["K"], p["G"]
    plain = fgg.rank_tiles(fgg.FP8, M, N, K, G, num_cus=fgg.device_info()["num_cus"])[0]["id"]
    aligned = fgg.rank_tiles(fgg.FP8, M, N, K, G, num_cus=fgg.device_info()["num_cus"],
                             run_align=128)[0]["id"]
    assert aligned != plain
    d = to_dev(p)
    fgg.tune_clear()
    log(f"run_align M={M} N={N} K={K} G={G} tiles {plain} -> {aligned}")
    c_al = run(p, d, run_align=128)
    assert np.array_equal(c_bits(c_al), c_bits(run(p, d, tile_id=aligned)))
    assert_parity(p, c_al)
    assert_parity(p, run(p, d))
    with pytest.raises(ValueError):
        run(p, d, run_align=-128)


def test_tune_takes_the_run_align_promise():
    """The tuning ranks its candidates under the caller's run_align promise:
    the first candidate is the aligned ranker's top tile, and the recorded
    choice matches the oracle."""
    counts = [128 * k for k in (5, 3, 9, 1, 6, 4, 2, 2)]
    p = fp8_problem(runs_to_indices(counts), 1024, 256, 8, np.random.default_rng(12))
    M, N, K, G = p["M"], p["N"], p["K"], p["G"]
    ncu = fgg.device_info()["num_cus"]
    aligned = [t["id"] for t in fgg.rank_tiles(fgg.FP8, M, N, K, G, num_cus=ncu, run_align=128)]
    d = to_dev(p)
    fgg.tune_clear()
    log(f"tune with run_align=128 M={M} N={N} K={K} G={G}")
    C, rep = _tune(p, d, top_k=2, reps=2, run_align=128)
    assert rep["tile_id"] == aligned[:2]
    assert_parity(p, C, what="tune with run_align")
    assert fgg.tuned_tile(fgg.FP8, M, N, K, G) == rep["chosen"]
    fgg.tune_clear()
