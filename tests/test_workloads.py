"""The seeded workloads: shapes, routing structure, determinism."""
import numpy as np
import pytest

from workloads import gen, make, runs_to_indices


def test_runs_to_indices():
    idx = runs_to_indices([3, 0, 2], pad_to=4, total=12)
    assert idx.tolist() == [0, 0, 0, -1, 2, 2, -1, -1, -1, -1, -1, -1]


def test_c1_routing():
    p = make("c1_tiny_fp8")
    assert (p["M"], p["N"], p["K"], p["G"]) == (256, 256, 512, 2)
    assert p["m_indices"].tolist() == [0] * 100 + [1] * 156
    assert p["A"].dtype == np.uint8 and p["A"].shape == (256, 512)
    assert p["a_scale"].shape == (256, 4) and p["b_scale"].shape == (2, 2, 4)
    assert np.all((p["A"] & 0x7F) != 0x7F)  # never a NaN code


def test_deterministic():
    a, b = make("p2_m777_g8"), make("p2_m777_g8")
    for k in ("A", "B", "a_scale", "b_scale", "m_indices"):
        assert np.array_equal(a[k], b[k])
    c = make("p2_m777_g8", seed=10)
    assert not np.array_equal(a["A"], c["A"])


def test_p2_shapes():
    p = make("p2_unaligned")
    assert (p["M"], p["N"], p["K"], p["G"]) == (65, 128, 128, 2)
    q = make("p2_m777_g8")
    assert (q["M"], q["N"], q["K"], q["G"]) == (777, 256, 512, 8)
    assert np.all(np.diff(q["m_indices"]) >= 0)


def test_window_runs_of_p2_shapes():
    """The flashinfer#7877 page launches ceil(M/128) * window_runs * ceil(N/64)
    CTAs, 4 for the M=65 shape and 84 for the M=777 one (section "Why it is
    good 1", table): window_runs 2 and 3.  The seed-9 routings reproduce
    those counts when window_runs is the largest number of distinct runs that
    meet one 128-row window."""
    def window_runs(ids):
        best = 0
        for w0 in range(0, ids.size, 128):
            win = ids[w0:w0 + 128]
            best = max(best, 1 + int(np.count_nonzero(win[1:] != win[:-1])))
        return best

    for name, ctas in (("p2_unaligned", 4), ("p2_m777_g8", 84)):
        p = make(name)
        n = -(-p["M"] // 128) * window_runs(p["m_indices"]) * -(-p["N"] // 64)
        assert n == ctas, name


@pytest.mark.slow
def test_c2_counts_and_shapes():
    p = make("c2_moe_fp8")
    counts = np.bincount(p["m_indices"], minlength=8)
    assert counts.tolist() == [1061, 1020, 1024, 1006, 1009, 1034, 973, 1065]
    assert p["B"].shape == (8, 4096, 7168) and p["b_scale"].shape == (8, 32, 56)


def test_c3_routing_only():
    rng = np.random.default_rng(0)
    counts = gen._zipf_counts(rng)
    idx = runs_to_indices(counts, pad_to=128, total=16384)
    assert idx.size == 16384
    assert int(np.count_nonzero(idx >= 0)) == 14336
    assert np.count_nonzero(counts) == 32
    # each expert's run starts on a 128-row boundary
    starts = np.nonzero(np.diff(np.concatenate([[-2], idx])) != 0)[0]
    for s in starts:
        if idx[s] >= 0:
            assert s % 128 == 0
    assert np.all(idx[-256:] == -1)


def test_nvfp4_small_problem_layout():
    rng = np.random.default_rng(0)
    p = gen.nvfp4_problem(None, 16, 128, 256, 1, rng)
    assert p["A"].shape == (16, 128) and p["a_scale"].shape == (16, 16)
    assert p["B"].shape == (128, 128) and p["b_scale"].shape == (128, 16)
    assert p["alpha"] == np.float32(p["gA"] * p["gB"])
