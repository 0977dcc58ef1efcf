"""GPU parity of grouped_w4a16_gemm (BF16 activations x NVFP4 weights, the
decode path of the onnxruntime#29824 page) against the float64 oracle,
through the C ABI.  Tolerance per BF16 element as for the other GEMMs:
|C - ref| <= 1e-2 |ref| + 1e-3 rms(ref); zero rows exactly zero."""
import numpy as np
import pytest

import oracle
import fp4_grouped_gemm_amd as fgg
from tests.gpu_util import c_bits, c_to_f64, log
from workloads import decode_routing, make, runs_to_indices, w4a16_problem

pytestmark = pytest.mark.gpu


def _dev(p):
    import torch
    A = torch.from_numpy(p["A_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    return dict(A=A, B=torch.from_numpy(p["B"]).cuda(), b_scale=torch.from_numpy(p["b_scale"]).cuda(),
                m_indices=torch.from_numpy(p["m_indices"]).cuda())


def _run(p, d=None):
    d = d or _dev(p)
    return fgg.grouped_w4a16_gemm(d["A"], d["B"], d["b_scale"], d["m_indices"], p["b_global"])


def _check(p, C, what, rows=None):
    ids = np.where((p["m_indices"] >= 0) & (p["m_indices"] < p["G"]), p["m_indices"], -1)
    ref = oracle.grouped_w4a16_gemm(p["A"], p["B"], p["b_scale"], ids, p["b_global"], rows=rows)
    out = c_to_f64(C)
    if rows is not None:
        out, ids = out[rows], ids[rows]
    res = oracle.check_tolerance(out, ref, ids)
    assert res["ok"], f"{what}: {res}"


def _prob(ids, N=256, K=512, G=None, seed=0):
    ids = np.asarray(ids, np.int32)
    G = G or max(1, int(ids.max()) + 1)
    return w4a16_problem(ids, N, K, G, np.random.default_rng(seed))


CASES = {
    "decode_top2": lambda: _prob(decode_routing(24, 2, 6, np.random.default_rng(1)), G=6, seed=1),
    "one_row": lambda: _prob([0], N=128, K=128),
    "padding_and_out_of_range": lambda: _prob([0, -1, 2, 9, 1, -7, 2, 2, -1, 0], G=3, seed=2),
    "empty_experts": lambda: _prob(runs_to_indices([0, 5, 0, 0, 40, 0]), G=6, seed=3),
    "more_than_16_rows": lambda: _prob(runs_to_indices([37, 70, 1]), N=384, K=384, seed=4),
    "K128_three_idle_waves": lambda: _prob([1, 0, 1, 1, 0], N=128, K=128, seed=5),
    "K_not_multiple_of_512": lambda: _prob([0, 1] * 9, N=256, K=640, seed=6),
    "rows_past_one_scan": lambda: _prob(np.random.default_rng(7).integers(-1, 2, 2500), N=128,
                                        K=256, G=2, seed=7),
    "single_expert": lambda: _prob([0] * 20, N=192 * 2, K=256, G=1, seed=8),
    # the scan bound: 1024 rows are one scan of m_indices, 1025 two (the
    # last row alone in the second), each with rows of every expert
    "scan_bound_1024": lambda: _prob(np.random.default_rng(9).integers(-1, 3, 1024), N=128,
                                     K=256, G=3, seed=9),
    "scan_bound_1025": lambda: _prob(np.random.default_rng(10).integers(-1, 3, 1025), N=128,
                                     K=256, G=3, seed=10),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_cases(case):
    p = CASES[case]()
    log(f"w4a16 {case} M={p['M']} N={p['N']} K={p['K']} G={p['G']}")
    _check(p, _run(p), case)


def test_deterministic_and_zero_rows_exact():
    p = CASES["padding_and_out_of_range"]()
    d = _dev(p)
    log("w4a16 determinism")
    a = c_bits(_run(p, d)).copy()
    b = c_bits(_run(p, d))
    assert np.array_equal(a, b)
    bad = (p["m_indices"] < 0) | (p["m_indices"] >= p["G"])
    assert np.all(a[bad] == 0)


@pytest.mark.slow
def test_full_size_decode():
    p = make("d5_decode_w4a16")
    log("w4a16 full-size decode")
    _check(p, _run(p), "d5_decode_w4a16")


def test_graph_replay_rereads_routing():
    """m_indices is read on the device at every launch: a captured call
    replayed after the routing changes gives the new routing's result."""
    import torch
    p = CASES["decode_top2"]()
    d = _dev(p)
    C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fgg.grouped_w4a16_gemm(d["A"], d["B"], d["b_scale"], d["m_indices"], p["b_global"], out=C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("w4a16 graph capture")
    with torch.cuda.graph(g):
        fgg.grouped_w4a16_gemm(d["A"], d["B"], d["b_scale"], d["m_indices"], p["b_global"], out=C)
    base = p["m_indices"]
    for rep, ids in enumerate([base, np.roll(base, 5), np.where(base % 2 == 0, -1, base)]):
        d["m_indices"].copy_(torch.from_numpy(ids.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(dict(p, m_indices=ids.astype(np.int32)), C, f"replay {rep}")
