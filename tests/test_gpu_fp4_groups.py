"""Grouped NVFP4 with a global scale per expert (grouped_fp4_gemm_alpha)
and batches of NVFP4 problems of different shapes in one launch
(fp4_gemm_problems), through the C ABI, against the float64 oracle
(cutlass#3124 page: grouped block-scaled GEMM over problems of different
M, N, K, with per-group scaling)."""
import numpy as np
import pytest

import oracle
import fp4_grouped_gemm_amd as fgg
from tests.gpu_util import assert_parity, c_bits, c_to_f64, log, to_dev
from workloads import nvfp4_problem, runs_to_indices

pytestmark = pytest.mark.gpu

TILES = [0, 1, 2, 3]


def _grouped(ids, N, K, G, seed):
    ids = np.asarray(ids, np.int32)
    return nvfp4_problem(ids, ids.size, N, K, G, np.random.default_rng(seed))


def _alpha_call(d, alphas_dev, **kw):
    return fgg.grouped_fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                                alphas_dev, **kw)


@pytest.mark.parametrize("tile", TILES)
def test_per_expert_alpha(tile):
    import torch
    p = _grouped(runs_to_indices([70, 0, 130, 57, 33], pad_to=8), 256, 512, 5, seed=21)
    alphas = np.array([0.5, 3.0, 1.0e-3, 7.25, 1.5e2], np.float32)
    d = to_dev(p)
    log(f"per-expert alpha tile {tile}")
    C = _alpha_call(d, torch.from_numpy(alphas).cuda(), tile_id=tile)
    assert_parity(dict(p, alpha=alphas), C, what=f"per-expert alpha tile {tile}")


def test_equal_per_expert_alphas_equal_the_scalar_call_bitwise():
    import torch
    p = _grouped(np.random.default_rng(22).integers(-1, 4, 301), 384, 256, 4, seed=22)
    d = to_dev(p)
    a = np.float32(p["alpha"])
    for tile in TILES:
        log(f"equal alphas tile {tile}")
        C1 = c_bits(fgg.grouped_fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"],
                                         d["m_indices"], float(a), tile_id=tile)).copy()
        C2 = c_bits(_alpha_call(d, torch.full((4,), float(a), device="cuda"), tile_id=tile))
        assert np.array_equal(C1, C2), tile


def test_per_expert_alpha_is_read_at_every_graph_replay():
    import torch
    p = _grouped(runs_to_indices([100, 60, 90]), 256, 256, 3, seed=23)
    d = to_dev(p)
    al = torch.ones(3, device="cuda")
    C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _alpha_call(d, al, out=C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("per-expert alpha graph capture")
    with torch.cuda.graph(g):
        _alpha_call(d, al, out=C)
    for vals in ([1.0, 1.0, 1.0], [0.25, 4.0, 2.0], [3.0, 0.5, 1.0]):
        al.copy_(torch.tensor(vals))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(dict(p, alpha=np.array(vals, np.float32)), C, what=f"replay {vals}")


def _problem(M, N, K, seed):
    return nvfp4_problem(None, M, N, K, 1, np.random.default_rng(seed))


BATCHES = {
    # different M, N and K in one launch; ragged M and N; one-row problem
    "mixed": [(200, 256, 512), (1, 128, 128), (333, 384, 1152), (64, 640, 256), (129, 128, 896)],
    "one": [(130, 256, 384)],
    "many_small": [(17 * (g + 1), 128 * (1 + g % 3), 128 * (1 + g % 4)) for g in range(12)],
}


def _run_batch(probs, **kw):
    ds = [to_dev(q) for q in probs]
    Cs = fgg.fp4_gemm_problems([(d["A"], d["B"], d["a_scale"], d["b_scale"], q["alpha"])
                                for d, q in zip(ds, probs)], **kw)
    return ds, Cs


@pytest.mark.parametrize("batch", sorted(BATCHES))
@pytest.mark.parametrize("tile", TILES)
def test_problem_batch(batch, tile):
    probs = [_problem(M, N, K, 30 + i) for i, (M, N, K) in enumerate(BATCHES[batch])]
    log(f"problem batch {batch} tile {tile}")
    _, Cs = _run_batch(probs, tile_id=tile)
    for i, (q, C) in enumerate(zip(probs, Cs)):
        assert_parity(q, C, what=f"{batch}/problem {i}/tile {tile}")


@pytest.mark.parametrize("max_wg", [1, 3])
def test_problem_batch_capped_grid(max_wg):
    probs = [_problem(M, N, K, 40 + i) for i, (M, N, K) in enumerate(BATCHES["mixed"])]
    for tile in TILES:
        log(f"problem batch capped grid max_wg={max_wg} tile {tile}")
        _, Cs = _run_batch(probs, tile_id=tile, max_workgroups=max_wg)
        for i, (q, C) in enumerate(zip(probs, Cs)):
            assert_parity(q, C, what=f"max_wg={max_wg}/problem {i}/tile {tile}")


def test_problem_in_a_batch_equals_fp4_gemm_bitwise():
    probs = [_problem(M, N, K, 50 + i) for i, (M, N, K) in enumerate(BATCHES["mixed"])]
    for tile in TILES:
        log(f"batch vs fp4_gemm tile {tile}")
        ds, Cs = _run_batch(probs, tile_id=tile)
        for d, q, C in zip(ds, probs, Cs):
            Cd = fgg.fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], q["alpha"], tile_id=tile)
            assert np.array_equal(c_bits(C), c_bits(Cd)), tile


@pytest.mark.slow
def test_full_size_problem_batch_sampled():
    """The 8-problem workload the benchmark times: every problem checked on
    its first, last and a seeded sample of rows."""
    from workloads import make
    p = make("p4_problems_nvfp4")
    probs = p["problems"]
    log("full-size problem batch")
    _, Cs = _run_batch(probs)
    rng = np.random.default_rng(5)
    for i, (q, C) in enumerate(zip(probs, Cs)):
        rows = np.unique(np.concatenate([[0, q["M"] - 1], rng.choice(q["M"], 24, replace=False)]))
        assert_parity(q, C, rows=rows, what=f"problem {i}")


def test_problem_batch_graph_replay():
    """The descriptors are kernel arguments, captured with the graph; new
    operand values written into the captured buffers are used at replay."""
    import torch
    shapes = BATCHES["mixed"]
    probs = [_problem(M, N, K, 60 + i) for i, (M, N, K) in enumerate(shapes)]
    ds = [to_dev(q) for q in probs]
    outs = [torch.empty((q["M"], q["N"]), dtype=torch.bfloat16, device="cuda") for q in probs]
    batch = [(d["A"], d["B"], d["a_scale"], d["b_scale"], q["alpha"]) for d, q in zip(ds, probs)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fgg.fp4_gemm_problems(batch, outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("problem batch graph capture")
    with torch.cuda.graph(g):
        fgg.fp4_gemm_problems(batch, outs)
    for rep in range(2):
        new = [_problem(M, N, K, 70 + 10 * rep + i) for i, (M, N, K) in enumerate(shapes)]
        for d, q in zip(ds, new):
            for k in ("A", "B", "a_scale", "b_scale"):
                d[k].copy_(torch.from_numpy(np.ascontiguousarray(q[k])))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (q, C) in enumerate(zip(new, outs)):
            # alpha is a captured kernel argument: the first batch's
            assert_parity(dict(q, alpha=probs[i]["alpha"]), C, what=f"replay {rep} problem {i}")
