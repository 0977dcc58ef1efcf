"""Batches of dense block-scaled FP8 problems of different shapes in one
launch (fp8_gemm_problems), through the C ABI, against the float64 oracle
(cutlass#3124 page, "Intro": grouped block-scaled GEMM over problems of
different M, N, K)."""
import numpy as np
import pytest

import fp4_grouped_gemm_amd as fgg
from tests.gpu_util import assert_parity, c_bits, log, to_dev
from workloads import fp8_problem

pytestmark = pytest.mark.gpu

TILES = [0, 1, 2, 3]


def _problem(M, N, K, seed):
    """A dense problem: every row routed to expert 0 of one."""
    return fp8_problem(np.zeros(M, np.int32), N, K, 1, np.random.default_rng(seed))


BATCHES = {
    # different M, N and K in one launch; ragged M; a one-row problem; K of
    # one, three and many 128-blocks
    "mixed": [(200, 256, 512), (1, 128, 128), (333, 384, 1152), (64, 640, 256), (129, 128, 896)],
    "one": [(130, 256, 384)],
    "many_small": [(17 * (g + 1), 128 * (1 + g % 3), 128 * (1 + g % 4)) for g in range(12)],
}


def _run_batch(probs, **kw):
    ds = [to_dev(q) for q in probs]
    Cs = fgg.fp8_gemm_problems([(d["A"], d["B"][0], d["a_scale"], d["b_scale"][0]) for d in ds],
                               **kw)
    return ds, Cs


@pytest.mark.parametrize("batch", sorted(BATCHES))
@pytest.mark.parametrize("tile", TILES)
def test_problem_batch(batch, tile):
    probs = [_problem(M, N, K, 60 + i) for i, (M, N, K) in enumerate(BATCHES[batch])]
    log(f"fp8 problem batch {batch} tile {tile}")
    _, Cs = _run_batch(probs, tile_id=tile)
    for i, (q, C) in enumerate(zip(probs, Cs)):
        assert_parity(q, C, what=f"{batch}/problem {i}/tile {tile}")


@pytest.mark.parametrize("max_wg", [1, 3])
def test_problem_batch_capped_grid(max_wg):
    """A capped persistent grid: each workgroup runs tiles of several
    problems back to back, restarting its pipeline state per tile."""
    probs = [_problem(M, N, K, 70 + i) for i, (M, N, K) in enumerate(BATCHES["mixed"])]
    for tile in TILES:
        log(f"fp8 problem batch capped grid max_wg={max_wg} tile {tile}")
        _, Cs = _run_batch(probs, tile_id=tile, max_workgroups=max_wg)
        for i, (q, C) in enumerate(zip(probs, Cs)):
            assert_parity(q, C, what=f"max_wg={max_wg}/problem {i}/tile {tile}")


def test_problem_in_a_batch_equals_grouped_call_bitwise():
    """Each problem of a batch gives the bits of grouped_fp8_gemm with G = 1
    and every row routed to expert 0, on the same tile config."""
    probs = [_problem(M, N, K, 80 + i) for i, (M, N, K) in enumerate(BATCHES["mixed"])]
    for tile in TILES:
        log(f"fp8 batch vs grouped call tile {tile}")
        ds, Cs = _run_batch(probs, tile_id=tile)
        for d, C in zip(ds, Cs):
            Cg = fgg.grouped_fp8_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                                      tile_id=tile, run_split=-1)
            assert np.array_equal(c_bits(C), c_bits(Cg)), tile


def test_problem_batch_ranker_choice():
    """No tile given: the ranker's choice over the summed terms."""
    probs = [_problem(M, N, K, 90 + i) for i, (M, N, K) in enumerate(BATCHES["many_small"])]
    log("fp8 problem batch, ranker's tile")
    _, Cs = _run_batch(probs)
    for i, (q, C) in enumerate(zip(probs, Cs)):
        assert_parity(q, C, what=f"ranker/problem {i}")


@pytest.mark.slow
def test_large_problem_batch_sampled():
    """Four problems of prefill size (the MoE layer's projections with
    different widths), each checked on its first, last and a seeded sample
    of rows."""
    shapes = [(2048, 4096, 7168), (1024, 2048, 7168), (4096, 1024, 2048), (333, 6144, 4096)]
    probs = [_problem(M, N, K, 100 + i) for i, (M, N, K) in enumerate(shapes)]
    log("fp8 large problem batch")
    _, Cs = _run_batch(probs)
    rng = np.random.default_rng(6)
    for i, (q, C) in enumerate(zip(probs, Cs)):
        rows = np.unique(np.concatenate([[0, q["M"] - 1], rng.choice(q["M"], 24, replace=False)]))
        assert_parity(q, C, rows=rows, what=f"problem {i}")


@pytest.mark.slow
def test_full_size_problem_batch_sampled():
    """The 8-problem workload the benchmark times: every problem checked on
    its first, last and a seeded sample of rows."""
    from workloads import make
    probs = make("p8_problems_fp8")["problems"]
    log("fp8 full-size problem batch")
    _, Cs = _run_batch(probs)
    rng = np.random.default_rng(7)
    for i, (q, C) in enumerate(zip(probs, Cs)):
        rows = np.unique(np.concatenate([[0, q["M"] - 1], rng.choice(q["M"], 24, replace=False)]))
        assert_parity(q, C, rows=rows, what=f"problem {i}")
