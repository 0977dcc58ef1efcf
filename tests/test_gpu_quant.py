"""GPU parity of the activation quantisers against the oracle (through the
C ABI).  Codes, scale codes and scales are integer / exact decisions taken in
FP32 on both sides, so every comparison is bitwise."""
import numpy as np
import pytest

import oracle.quant as oq
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _bf16(rng, M, K, scale=1.0, dist="normal"):
    """Seeded BF16-representable float32 values (and the bf16 tensor)."""
    import torch
    if dist == "student_t3":
        x = rng.standard_t(3, (M, K))
    else:
        x = rng.standard_normal((M, K))
    x = (x * scale).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.float().numpy(), t


def _gpu_fp8(t):
    import fp4_grouped_gemm_amd as fgg
    Q, S = fgg.quantize_fp8_1x128(t.cuda())
    return Q.cpu().numpy(), S.cpu().numpy()


def _gpu_nvfp4(t):
    import fp4_grouped_gemm_amd as fgg
    Q, S, g = fgg.quantize_nvfp4(t.cuda())
    return Q.cpu().numpy(), S.cpu().numpy(), np.float32(g.cpu().numpy()[0])


CASES = {
    "small": (3, 128, 1.0, "normal"),
    "ragged_rows": (37, 384, 3.0, "normal"),
    "wide": (5, 4224, 0.01, "normal"),
    "heavy_tail": (64, 1024, 1.0, "student_t3"),
    "tiny_values": (16, 256, 1e-30, "normal"),
    "big_values": (16, 256, 1e30, "normal"),
    "one_row": (1, 7168, 1.0, "normal"),
    "odd_segments": (3, 640, 2.0, "normal"),  # 15 blocks of 128: a partial wave segment
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_1x128_bitwise(case):
    M, K, sc, dist = CASES[case]
    x, t = _bf16(np.random.default_rng(100 + sorted(CASES).index(case)), M, K, sc, dist)
    x[:, :128][0] = 0.0  # an all-zero block in the first row
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    log(f"quantize_fp8_1x128 {case} M={M} K={K}")
    Q, S = _gpu_fp8(t)
    q_ref, s_ref = oq.quantize_fp8_1x128(x)
    assert np.array_equal(S.view(np.uint32), s_ref.view(np.uint32)), case
    assert np.array_equal(Q, q_ref), (case, int((Q != q_ref).sum()))


@pytest.mark.parametrize("case", sorted(CASES))
def test_nvfp4_bitwise(case):
    M, K, sc, dist = CASES[case]
    x, t = _bf16(np.random.default_rng(200 + sorted(CASES).index(case)), M, K, sc, dist)
    x[0, 16:48] = 0.0  # all-zero 16-blocks
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    log(f"quantize_nvfp4 {case} M={M} K={K}")
    Q, S, g = _gpu_nvfp4(t)
    q_ref, s_ref, g_ref = oq.quantize_nvfp4(x)
    assert g == g_ref, (case, g, g_ref)
    assert np.array_equal(S, s_ref), (case, int((S != s_ref).sum()))
    assert np.array_equal(Q, q_ref), (case, int((Q != q_ref).sum()))


STATIC_G = {
    "dynamic": None,       # g = amax / 2688, as the dynamic quantiser takes it
    "saturating": 1 / 64,  # the dynamic g / 64: large blocks clamp at s = 448, codes at 6
    "odd": 0.7654321,      # not a power of two
    "min_normal": float(np.finfo(np.float32).tiny),  # every nonzero block saturates
    "huge": 1e30,          # most blocks underflow to s = 0 and zero codes
}


@pytest.mark.parametrize("gname", sorted(STATIC_G))
@pytest.mark.parametrize("case", ["ragged_rows", "heavy_tail", "one_row", "odd_segments"])
def test_nvfp4_static_scale_bitwise(case, gname):
    """The given-global-scale quantiser against the oracle with that g."""
    import torch
    import fp4_grouped_gemm_amd as fgg
    M, K, sc, dist = CASES[case]
    x, t = _bf16(np.random.default_rng(300 + sorted(CASES).index(case)), M, K, sc, dist)
    x[0, 16:48] = 0.0
    t = torch.from_numpy(x).to(torch.bfloat16)
    g_dyn = oq.quantize_nvfp4(x)[2]
    g = STATIC_G[gname]
    g = float(g_dyn) if g is None else (float(g_dyn) * g if gname == "saturating" else g)
    log(f"quantize_nvfp4_static {case} g={gname} M={M} K={K}")
    Q, S, gt = fgg.quantize_nvfp4(t.cuda(), global_scale=g)
    Q, S = Q.cpu().numpy(), S.cpu().numpy()
    q_ref, s_ref, g_ref = oq.quantize_nvfp4(x, g)
    assert np.float32(gt.cpu().numpy()[0]) == g_ref
    assert np.array_equal(S, s_ref), (case, gname, int((S != s_ref).sum()))
    assert np.array_equal(Q, q_ref), (case, gname, int((Q != q_ref).sum()))
    if gname == "dynamic":  # same g, same bits as the amax-pass quantiser
        Qd, Sd, _ = _gpu_nvfp4(t)
        assert np.array_equal(Q, Qd) and np.array_equal(S, Sd)
    if gname == "saturating":
        assert (s_ref == 0x7E).any()  # the clamp was reached (E4M3FN 448)


def test_every_bf16_value_through_fp8():
    """Every finite BF16 bit pattern as an element next to a block maximum
    of 448 (scale 1.0): each code is the E4M3FN rounding of the value itself
    (covers rounding, ties, subnormals, signed zero and clamping)."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    n = -(-v.size // 127) * 127
    vals = np.zeros(n, np.float32)
    vals[:v.size] = v
    blocks = vals.reshape(-1, 127)
    x = np.concatenate([np.full((blocks.shape[0], 1), 448.0, np.float32), blocks], axis=1)
    x = x.reshape(-1, 128 * 8) if x.shape[0] % 8 == 0 else x.reshape(-1, 128)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), x)
    log(f"every bf16 value through fp8: {v.size} values")
    Q, S = _gpu_fp8(t)
    q_ref, s_ref = oq.quantize_fp8_1x128(x)
    assert np.all(S == 1.0)
    assert np.array_equal(Q, q_ref), int((Q != q_ref).sum())


def _bf16_values(limit):
    """Every finite BF16 value of magnitude <= limit, as float32."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v) & (np.abs(v) <= limit)]


@pytest.mark.parametrize("lead", [613.0, 301.0, 1.7e-5, 3.3e20])
def test_every_bf16_value_through_fp8_odd_scale(lead):
    """Every BF16 value up to a block maximum whose scale (lead / 448) is not
    a power of two: each code follows the IEEE quotient x / scale."""
    import torch
    lead = float(torch.tensor(lead).to(torch.bfloat16).float())
    v = _bf16_values(lead)
    n = -(-v.size // 127) * 127
    vals = np.zeros(n, np.float32)
    vals[:v.size] = v
    x = np.concatenate([np.full((n // 127, 1), lead, np.float32), vals.reshape(-1, 127)], axis=1)
    x = x.reshape(-1, 128)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), x)
    log(f"every bf16 value through fp8, block max {lead}: {v.size} values")
    Q, S = _gpu_fp8(t)
    q_ref, s_ref = oq.quantize_fp8_1x128(x)
    assert np.array_equal(S.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(Q, q_ref), int((Q != q_ref).sum())


@pytest.mark.parametrize("g", [0.7654321, 3.1e-7, 1.3e9])
def test_every_bf16_value_through_nvfp4_odd_scale(g):
    """Every BF16 value up to 6 * 448 * g in blocks led by values that give
    scale codes of every size, with a static global scale that is not a power
    of two: each code follows the IEEE quotient x / (value(s) g)."""
    import torch
    import fp4_grouped_gemm_amd as fgg
    g = float(np.float32(g))
    v = _bf16_values(6 * 448 * g)
    rng = np.random.default_rng(7)
    leads = np.abs(rng.choice(v, size=-(-v.size // 15)))
    n = leads.size * 15
    vals = np.zeros(n, np.float32)
    vals[:v.size] = v
    blocks = vals.reshape(-1, 15)
    blocks = np.clip(blocks, -leads[:, None], leads[:, None])  # the lead is the block maximum
    x = np.concatenate([leads[:, None].astype(np.float32), blocks], axis=1)
    rows = -(-x.shape[0] // 8)
    x = np.concatenate([x, np.zeros((rows * 8 - x.shape[0], 16), np.float32)]).reshape(rows, 128)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), x)
    log(f"every bf16 value through nvfp4, static g {g}: {x.size} values")
    Q, S, _ = fgg.quantize_nvfp4(t.cuda(), global_scale=g)
    q_ref, s_ref, _ = oq.quantize_nvfp4(x, g)
    assert np.array_equal(S.cpu().numpy(), s_ref)
    assert np.array_equal(Q.cpu().numpy(), q_ref), int((Q.cpu().numpy() != q_ref).sum())


def test_every_fp4_rounding_case():
    """Values on a 1/64 grid through [-6.5, 6.5], each 16-block led by 6.0,
    with the tensor maximum 2688: g = 1, every such block gets s = 1.0 and
    d = 1, so each code is the E2M1 rounding of the value itself (ties,
    signed zero and clamping included)."""
    import torch
    grid = (np.arange(-6.5 * 64, 6.5 * 64 + 1) / 64).astype(np.float32)
    n = -(-grid.size // 15) * 15
    vals = np.zeros(n, np.float32)
    vals[:grid.size] = grid
    blocks = vals.reshape(-1, 15)
    x = np.concatenate([np.full((blocks.shape[0], 1), 6.0, np.float32), blocks], axis=1)
    rows = -(-x.shape[0] // 8)
    pad = np.zeros((rows * 8 - x.shape[0], 16), np.float32)
    x = np.concatenate([x, pad]).reshape(rows, 128)
    x[0, 0] = 2688.0  # tensor amax: g = 1
    t = torch.from_numpy(x).to(torch.bfloat16)
    x = t.float().numpy()
    log("fp4 rounding grid")
    Q, S, g = _gpu_nvfp4(t)
    q_ref, s_ref, g_ref = oq.quantize_nvfp4(x)
    assert g == g_ref == 1.0
    assert np.array_equal(S, s_ref)
    assert np.array_equal(Q, q_ref), int((Q != q_ref).sum())


def test_quantised_activations_feed_the_gemm():
    """quantize_fp8_1x128 output is a valid A operand: the grouped FP8 GEMM on
    it matches the oracle GEMM on the oracle-quantised A."""
    import torch

    import fp4_grouped_gemm_amd as fgg
    import oracle
    from workloads import runs_to_indices
    rng = np.random.default_rng(21)
    M, N, K, G = 300, 256, 512, 3
    x, t = _bf16(rng, M, K)
    ids = runs_to_indices([100, 0, 200], pad_to=1)
    from workloads import fp8_problem
    p = fp8_problem(ids, N, K, G, rng)
    Q, S = fgg.quantize_fp8_1x128(t.cuda())
    C = fgg.grouped_fp8_gemm(Q, torch.from_numpy(p["B"]).cuda(), S,
                             torch.from_numpy(p["b_scale"]).cuda(),
                             torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = oq.quantize_fp8_1x128(x)
    ref = oracle.grouped_fp8_gemm(q_ref, p["B"], s_ref, p["b_scale"], ids)
    out = C.float().cpu().numpy().astype(np.float64)
    res = oracle.check_tolerance(out, ref, ids)
    assert res["ok"], res


EDGE = {
    "one_block": (1, 128),        # 4 of 64 lanes hold a piece (FP8), 4 blocks (NVFP4)
    "one_wave_plus_one": (1, 2176),  # 17 FP8 blocks, 136 NVFP4 blocks
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_partial_waves_bitwise(case):
    M, K = EDGE[case]
    x, t = _bf16(np.random.default_rng(300 + sorted(EDGE).index(case)), M, K)
    log(f"quantisers partial wave {case}")
    Q, S = _gpu_fp8(t)
    q_ref, s_ref = oq.quantize_fp8_1x128(x)
    assert np.array_equal(Q, q_ref) and np.array_equal(S, s_ref)
    Q, S, g = _gpu_nvfp4(t)
    q_ref, s_ref, g_ref = oq.quantize_nvfp4(x)
    assert g == g_ref and np.array_equal(Q, q_ref) and np.array_equal(S, s_ref)


def test_all_zero_input():
    import torch
    t = torch.zeros((4, 256), dtype=torch.bfloat16)
    log("quantisers all-zero input")
    Q, S = _gpu_fp8(t)
    assert not Q.any() and np.all(S == 1.0)
    Q, S, g = _gpu_nvfp4(t)
    assert not Q.any() and not S.any() and g == 1.0


def test_graph_replay_with_new_inputs():
    """Both quantisers captured in one HIP graph (the NVFP4 path is four
    kernels, no memset node) and replayed on new data written into the
    captured input, each replay bitwise against the oracle."""
    import torch
    import fp4_grouped_gemm_amd as fgg
    M, K = 24, 1152
    X = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    X.copy_(_bf16(np.random.default_rng(400), M, K)[1])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fgg.quantize_fp8_1x128(X)
        fgg.quantize_nvfp4(X)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("quantisers graph capture")
    with torch.cuda.graph(g):
        q8, s8 = fgg.quantize_fp8_1x128(X)
        q4, s4, g4 = fgg.quantize_nvfp4(X)
    for rep in range(3):
        x, t = _bf16(np.random.default_rng(401 + rep), M, K, scale=10.0 ** (rep - 1))
        X.copy_(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r8 = oq.quantize_fp8_1x128(x)
        r4 = oq.quantize_nvfp4(x)
        assert np.array_equal(q8.cpu().numpy(), r8[0]) and np.array_equal(s8.cpu().numpy(), r8[1])
        assert np.float32(g4.cpu().numpy()[0]) == r4[2], rep
        assert np.array_equal(q4.cpu().numpy(), r4[0]) and np.array_equal(s4.cpu().numpy(), r4[1])


@pytest.mark.slow
def test_grid_stride_loops_on_sampled_rows():
    """A tensor large enough that every wave of the capped grids takes
    several turns of its loop; rows are independent (FP8) or share only the
    global scale (NVFP4), so sampled rows are checked against the oracle."""
    import torch
    M, K = 16384, 8192
    rng = np.random.default_rng(500)
    t = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16)
    x = t.float().numpy()
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    log("quantisers grid-stride loops")
    Q, S = _gpu_fp8(t)
    q_ref, s_ref = oq.quantize_fp8_1x128(x[rows])
    assert np.array_equal(Q[rows], q_ref) and np.array_equal(S[rows], s_ref)
    Q, S, g = _gpu_nvfp4(t)
    g_ref = oq.nvfp4_global_scale(x)
    assert g == g_ref
    q_ref, s_ref, _ = oq.quantize_nvfp4(x[rows], g_ref)
    assert np.array_equal(Q[rows], q_ref) and np.array_equal(S[rows], s_ref)


@pytest.mark.slow
def test_bench_shapes_sampled():
    """The bench's quantiser workloads at full size, as it launches them
    (seeded N(0,1) BF16 activations: c2's A 8192 x 7168 through FP8, c5's A
    65536 x 8192 through NVFP4 with the computed and with a calibrated global
    scale): sampled rows bitwise against the oracle, the global scale exact."""
    import torch
    import fp4_grouped_gemm_amd as fgg
    for M, K, fmt in ((8192, 7168, "fp8"), (65536, 8192, "nvfp4")):
        rng = np.random.default_rng(0)
        t = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16)
        rows = np.unique(np.concatenate([[0, 1, M - 1], rng.choice(M, 40, replace=False)]))
        xs = t[torch.from_numpy(rows)].float().numpy()
        log(f"quantiser {fmt} full size M={M} K={K}")
        if fmt == "fp8":
            Q, S = _gpu_fp8(t)
            q_ref, s_ref = oq.quantize_fp8_1x128(xs)
            assert np.array_equal(Q[rows], q_ref) and np.array_equal(S[rows], s_ref)
            continue
        Q, S, g = _gpu_nvfp4(t)
        amax = np.float32(float(t.cuda().float().abs().max()))  # the tensor's maximum, exactly
        g_ref = oq.nvfp4_global_scale(np.array([amax], np.float32))
        assert g == g_ref
        q_ref, s_ref, _ = oq.quantize_nvfp4(xs, g_ref)
        assert np.array_equal(Q[rows], q_ref) and np.array_equal(S[rows], s_ref)
        g_static = float(t[:64].float().abs().max()) / 2688.0  # the bench's calibration
        Qs, Ss, _ = fgg.quantize_nvfp4(t.cuda(), global_scale=g_static)
        q_ref, s_ref, _ = oq.quantize_nvfp4(xs, np.float32(g_static))
        assert np.array_equal(Qs.cpu().numpy()[rows], q_ref)
        assert np.array_equal(Ss.cpu().numpy()[rows], s_ref)
