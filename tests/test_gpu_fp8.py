"""GPU parity of grouped_fp8_gemm against the float64 oracle (through the
C ABI).  Tolerance per BF16 element: |C - ref| <= 1e-2 |ref| + 1e-3 rms(ref);
padding rows exactly zero; exact cases bitwise."""
import numpy as np
import pytest

from tests.golden_build import build, load_examples
from tests.gpu_util import (assert_parity, c_bits, c_to_f64, log, ref, row_ids, run,
                            sample_rows, to_dev)
from workloads import fp8_problem, make, runs_to_indices

pytestmark = pytest.mark.gpu

FP8_TILES = [0, 1, 2, 3]


@pytest.mark.parametrize("ex", [e for e in load_examples() if e["kind"] == "fp8"],
                         ids=lambda e: e["name"])
def test_worked_examples_bitwise(ex):
    d = build(ex)
    for tile in FP8_TILES:
        log(f"worked example {ex['name']} tile {tile}")
        C = run(d, tile_id=tile)
        assert np.array_equal(c_bits(C), d["expected_bf16"]), (ex["name"], tile)


@pytest.mark.parametrize("name", ["c1_tiny_fp8", "p2_unaligned", "p2_m777_g8"])
@pytest.mark.parametrize("tile", FP8_TILES)
def test_small_configs_all_tiles(name, tile):
    p = make(name)
    log(f"{name} tile {tile}")
    C = run(p, tile_id=tile)
    assert_parity(p, C, what=f"{name}/tile{tile}")


def _prob(ids, N=256, K=512, G=None, seed=0, **kw):
    ids = np.asarray(ids, np.int32)
    G = G or max(1, int(ids.max()) + 1)
    return fp8_problem(ids, N, K, G, np.random.default_rng(seed), **kw)


EDGE = {
    "M1": lambda: _prob([0]),
    "all_padding": lambda: _prob([-1] * 300, G=3),
    "run_of_one": lambda: _prob([0] * 50 + [1] + [2] * 100, G=3),
    "run_across_windows": lambda: _prob([0] * 3 + [1] * 600 + [2] * 5, G=3),
    "empty_experts": lambda: _prob(runs_to_indices([0, 70, 0, 0, 200, 0]), G=6),
    "single_expert": lambda: _prob([0] * 513, G=1),
    "unsorted_rows": lambda: _prob(np.random.default_rng(4).integers(-1, 5, 333), G=5),
    "out_of_range_ids": lambda: _prob([0, 7, -5, 1, 2, 1 << 30, -1, 0] * 40, G=3),
    "many_experts_one_window": lambda: _prob(np.arange(40) % 20, G=20),
    # more experts than tile rows: split mode's item r runs expert r, so items
    # past the tile height must find their rows too
    "more_experts_than_rows": lambda: _prob(np.random.default_rng(11).integers(-1, 300, 400), G=300),
    "K128_N128": lambda: _prob([0] * 10 + [1] * 10, N=128, K=128),
    "N_not_tile_multiple": lambda: _prob([0] * 100 + [1] * 200, N=384, K=256),
    # K steps a multiple of the 3-stage loop's six-step unroll, and an odd
    # count below it, each with a run boundary inside a window
    "K768_six_steps": lambda: _prob([0] * 70 + [1] * 90, K=768),
    "K384_three_steps": lambda: _prob([0] * 130 + [1] * 70, K=384),
}


@pytest.mark.parametrize("case", sorted(EDGE))
@pytest.mark.parametrize("tile", FP8_TILES)
def test_edge_cases(case, tile):
    p = EDGE[case]()
    log(f"edge {case} tile {tile} M={p['M']} N={p['N']} K={p['K']} G={p['G']}")
    C = run(p, tile_id=tile)
    assert_parity(p, C, what=f"{case}/tile{tile}")


SPLIT_CASES = ["run_of_one", "run_across_windows", "empty_experts", "unsorted_rows",
               "out_of_range_ids", "many_experts_one_window", "all_padding", "N_not_tile_multiple",
               "more_experts_than_rows"]


@pytest.mark.parametrize("case", SPLIT_CASES + ["p2_m777_g8", "c1_tiny_fp8"])
def test_run_split_modes_agree_bitwise(case):
    """Each expert pass of a window as its own workgroup (run_split=1) or
    all passes in one workgroup (-1): the same arithmetic in the same order,
    so the same bits, and both within the oracle's tolerance."""
    p = EDGE[case]() if case in EDGE else make(case)
    d = to_dev(p)
    for tile in FP8_TILES:
        log(f"run split {case} tile {tile}")
        split = c_bits(run(p, d, tile_id=tile, run_split=1)).copy()
        C = run(p, d, tile_id=tile, run_split=-1)
        assert np.array_equal(split, c_bits(C)), (case, tile)
        assert_parity(p, C, what=f"split {case}/tile{tile}")


@pytest.mark.parametrize("max_wg", [1, 5])
def test_run_split_with_capped_grid(max_wg):
    """Split items on a capped persistent grid: a workgroup runs passes of
    many tiles back to back."""
    p = EDGE["many_experts_one_window"]()
    for tile in FP8_TILES:
        log(f"run split capped grid max_wg={max_wg} tile {tile}")
        C = run(p, tile_id=tile, run_split=1, max_workgroups=max_wg)
        assert_parity(p, C, what=f"split max_wg={max_wg}/tile{tile}")


@pytest.mark.parametrize("max_wg", [1, 3, 7])
def test_persistent_loop_reinitialises_state(max_wg):
    """A capped grid makes each workgroup run many tiles and passes back to
    back; every tile must restart its pipeline state (the stale-token
    lesson of the cutlass#3124 page, "Code analysis 2")."""
    p = make("p2_m777_g8")
    for tile in FP8_TILES:
        log(f"persistent max_wg={max_wg} tile {tile}")
        C = run(p, tile_id=tile, max_workgroups=max_wg)
        assert_parity(p, C, what=f"max_wg={max_wg}/tile{tile}")


@pytest.mark.parametrize("K", [8320, 16640])
def test_long_k_b_scale_per_block(K):
    """K above 64 scale blocks: the kernel holds a wave's b_scale row 64
    blocks at a time and reloads the next 64 in the loop.  b_scale varies by
    powers of two from block to block, so a block read from the wrong
    position would be far outside the tolerance."""
    p = _prob([0] * 70 + [1] * 90, N=256, K=K, G=2, seed=21)
    rng = np.random.default_rng(22)
    p["b_scale"] = (p["b_scale"] * np.exp2(rng.integers(-6, 7, p["b_scale"].shape))
                    ).astype(np.float32)
    for tile in FP8_TILES:
        log(f"long K={K} tile {tile}")
        C = run(p, tile_id=tile)
        assert_parity(p, C, what=f"K={K}/tile{tile}")


def test_small_integer_inputs_bitwise():
    """Codes decoding to small integers and power-of-two scales keep every
    FP32 operation exact, so the BF16 output must equal the oracle's
    round-to-nearest-even bitwise."""
    import oracle
    rng = np.random.default_rng(8)
    ids = runs_to_indices([37, 0, 150, 69], pad_to=1)
    M, N, K, G = ids.size, 256, 384, 4
    small = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50,
                      0xB8, 0xC0, 0xC4, 0xC8, 0xCA, 0xCC, 0xCE, 0xD0], np.uint8)  # 0, +-1..8
    p = dict(kind="fp8", M=M, N=N, K=K, G=G, m_indices=ids,
             A=rng.choice(small, (M, K)), B=rng.choice(small, (G, N, K)),
             a_scale=np.exp2(rng.integers(-3, 4, (M, K // 128))).astype(np.float32),
             b_scale=np.exp2(rng.integers(-3, 4, (G, N // 128, K // 128))).astype(np.float32))
    want = oracle.bf16_rne_bits(ref(p))
    for tile in FP8_TILES:
        log(f"small-integer bitwise tile {tile}")
        assert np.array_equal(c_bits(run(p, tile_id=tile)), want), tile


def test_deterministic_and_guard_bands():
    import torch
    p = make("p2_m777_g8")
    d = to_dev(p)
    M, N = p["M"], p["N"]
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), 0x7FBF, dtype=torch.int16, device="cuda")
    out = buf[pad:pad + M * N].view(torch.bfloat16).view(M, N)
    log("guard bands")
    run(p, d, out=out)
    torch.cuda.synchronize()
    guard = buf.cpu().numpy()
    assert np.all(guard[:pad] == 0x7FBF) and np.all(guard[-pad:] == 0x7FBF)
    first = c_bits(out).copy()
    second = c_bits(run(p, d))
    assert np.array_equal(first, second)


def test_graph_replay_rereads_m_indices():
    """m_indices is read on the device at every launch, so a captured graph
    replayed after the routing changes gives the new routing's result
    (flashinfer#7877 page, "Code analysis 2")."""
    import torch
    p = make("p2_m777_g8")
    d = to_dev(p)
    C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(p, d, out=C)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("graph capture")
    with torch.cuda.graph(g):
        run(p, d, out=C)
    routings = [p["m_indices"], np.roll(p["m_indices"], 37), np.where(p["m_indices"] % 3 == 0, -1,
                                                                      p["m_indices"])]
    for rep in range(2):
        for r in routings:
            d["m_indices"].copy_(torch.from_numpy(r.astype(np.int32)))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            q = dict(p, m_indices=r.astype(np.int32))
            assert_parity(q, C, what=f"graph replay {rep}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c2_moe_fp8", "c3_skewed_fp8"])
def test_full_size_sampled(name):
    p = make(name)
    d = to_dev(p)
    rows = sample_rows(p, 384)
    log(f"{name} full size, ranker's tile")
    C = run(p, d)
    assert_parity(p, C, rows=rows, what=name)
    out = c_to_f64(C)
    ids = row_ids(p)
    assert np.all(out[ids < 0] == 0.0)  # every padding row, not only the sample
    assert np.all(np.isfinite(out))
    # Every tile shape accumulates and promotes each output over the same K
    # blocks in the same order, so all of them give the same bits: compared
    # on every element, and each against the oracle on a sample of rows.
    bits = c_bits(C).copy()
    for tile in FP8_TILES:
        log(f"{name} full size tile {tile}")
        C = run(p, d, tile_id=tile)
        assert_parity(p, C, rows=rows[::3], what=f"{name}/tile{tile}")
        assert np.array_equal(c_bits(C), bits), (name, tile)
    if name == "c3_skewed_fp8":  # as the bench launches it: runs padded to 128, promised
        log(f"{name} full size, run_align=128")
        C = run(p, d, run_align=128)
        assert_parity(p, C, rows=rows, what=f"{name}/run_align")
        assert np.all(c_to_f64(C)[ids < 0] == 0.0)


@pytest.mark.slow
def test_more_windows_than_the_tile_plan_tracks():
    """Past 4096 row windows the heavy-first tile order is not built and
    tiles go in the plain XCD order; 128-row windows of 600000 rows exceed
    that.  Sampled rows against the oracle, every padding row zero."""
    rng = np.random.default_rng(11)
    counts = rng.integers(0, 40000, 24)
    counts[5] = 0
    ids = runs_to_indices(counts.tolist(), pad_to=1)
    ids = np.concatenate([ids, np.full(600000 - ids.size, -1, np.int32)]) if ids.size < 600000 \
        else ids[:600000]
    p = _prob(ids, N=128, K=128, G=24, seed=12)
    d = to_dev(p)
    rows = sample_rows(p, 256)
    for tile in (3, 0):
        log(f"600000 rows, tile {tile}")
        C = run(p, d, tile_id=tile)
        assert_parity(p, C, rows=rows, what=f"many windows/tile{tile}")
        out = c_to_f64(C)
        assert np.all(out[row_ids(p) < 0] == 0.0)


def test_every_e4m3_code_exact():
    """All 254 non-NaN E4M3 codes of A against an identity B: each output is
    one product decode(A[i, n]) * 1.0, exact in BF16, so it must match the
    oracle bitwise (pins the device's E4M3FN decode, including subnormals
    and the 448 maximum)."""
    import oracle
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    K = N = 128
    M = -(-codes.size // K)
    A = np.zeros((M, K), np.uint8)
    A.flat[:codes.size] = codes
    B = np.where(np.eye(N, K, dtype=bool), 0x38, 0x00).astype(np.uint8)[None]
    p = dict(kind="fp8", M=M, N=N, K=K, G=1, A=A, B=B, m_indices=np.zeros(M, np.int32),
             a_scale=np.ones((M, 1), np.float32), b_scale=np.ones((1, 1, 1), np.float32))
    want = oracle.bf16_rne_bits(ref(p))
    for tile in FP8_TILES:
        log(f"exhaustive e4m3 tile {tile}")
        assert np.array_equal(c_bits(run(p, tile_id=tile)), want), tile
