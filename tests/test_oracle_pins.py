"""Pins of the oracle's GEMMs against things other than itself.

* exact brute force: E4M3 values are integers times 2^-9, E2M1 values are
  integers times 2^-1, so block partial sums are exact in int64 and the whole
  result is an exact rational (fractions.Fraction) -- computed here with an
  integer decode written independently of the oracle's;
* the hand-computed worked examples in tests/golden;
* invariants of the definition (padding rows, expert relabelling, row
  permutation, power-of-two scale changes, sign flips, zero scales, G = 1);
* a special case that reduces to a library routine: with unit scales and one
  expert the result is a plain float64 matmul of PyTorch-decoded FP8 values.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.golden_build import build, load_examples
from workloads import fp8_problem, nvfp4_problem, runs_to_indices


# ---------------------------------------------------------------- brute force
def _e4m3_int_table():
    t = np.zeros(256, np.int64)
    for c in range(256):
        s = -1 if c & 0x80 else 1
        E, M = (c >> 3) & 15, c & 7
        t[c] = 0 if (E == 15 and M == 7) else s * (M if E == 0 else (8 + M) << (E - 1))
    return t  # value = t * 2^-9


def _e2m1_int_table():
    t = np.zeros(16, np.int64)
    for c in range(16):
        s = -1 if c & 8 else 1
        E, M = (c >> 1) & 3, c & 1
        t[c] = s * (M if E == 0 else (2 + M) << (E - 1))
    return t  # value = t * 2^-1


def brute_fp8(A, B, a_scale, b_scale, ids):
    """Exact C as Fractions, plus sum of |terms| for the rounding bound."""
    T = _e4m3_int_table()
    Ai, Bi = T[A], T[B]
    M, K = A.shape
    G, N, _ = B.shape
    C = [[Fraction(0)] * N for _ in range(M)]
    mag = np.zeros((M, N))
    for i in range(M):
        g = int(ids[i])
        if g < 0:
            continue
        for kb in range(K // 128):
            ks = slice(kb * 128, kb * 128 + 128)
            P = Bi[g][:, ks] @ Ai[i, ks]  # exact int64 partials, one per column
            fa = Fraction(float(a_scale[i, kb]))
            for n in range(N):
                t = fa * Fraction(float(b_scale[g, n // 128, kb])) * int(P[n]) / (1 << 18)
                C[i][n] += t
                mag[i, n] += abs(float(t))
    return C, mag


def brute_nvfp4(A, B, a_sc, b_sc, ids, alpha):
    """Exact C / alpha as an int64 multiple of 2^-20 (E2M1 2^-1 twice, E4M3 2^-9 twice)."""
    Q, S = _e2m1_int_table(), _e4m3_int_table()

    def unpack(p):
        out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
        out[..., 0::2], out[..., 1::2] = p & 0xF, p >> 4
        return out

    qa, qb = Q[unpack(A)], Q[unpack(B)]
    sa, sb = S[a_sc], S[b_sc]
    M, K = qa.shape
    if ids is None:
        qb, sb, ids = qb[None], sb[None], np.zeros(M, np.int32)
    N = qb.shape[1]
    tot = np.zeros((M, N), np.int64)
    for i in range(M):
        g = int(ids[i])
        if g < 0:
            continue
        for blk in range(K // 16):
            ks = slice(blk * 16, blk * 16 + 16)
            part = qb[g][:, ks] @ qa[i, ks]
            tot[i] += part * sb[g][:, blk] * sa[i, blk]
    return tot


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_oracle_equals_exact_rational(seed):
    rng = np.random.default_rng(100 + seed)
    ids = np.array([2, 2, 0, -1, 1, 1, 1, 2, -1, 0, 0, 2], np.int32)
    p = fp8_problem(ids, 256, 384, 3, rng)
    # spread the scales over many binades so a wrong index changes the result
    p["a_scale"] *= np.exp2(rng.integers(-6, 7, p["a_scale"].shape)).astype(np.float32)
    p["b_scale"] *= np.exp2(rng.integers(-6, 7, p["b_scale"].shape)).astype(np.float32)
    C = oracle.grouped_fp8_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], ids)
    exact, mag = brute_fp8(p["A"], p["B"], p["a_scale"], p["b_scale"], ids)
    nkb = 384 // 128
    for i in range(len(ids)):
        for n in range(256):
            bound = 4 * nkb * 2.0 ** -53 * mag[i, n]
            assert abs(C[i, n] - float(exact[i][n])) <= bound + 1e-300, (i, n)
    assert np.all(C[ids == -1] == 0.0)


@pytest.mark.parametrize("grouped", [False, True])
def test_nvfp4_oracle_equals_exact_integer(grouped):
    rng = np.random.default_rng(7)
    if grouped:
        ids = np.array([1, 0, -1, 1, 2, 2, 0], np.int32)
        p = nvfp4_problem(ids, 7, 128, 256, 3, rng)
        C = oracle.grouped_fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], ids, p["alpha"])
    else:
        ids = None
        p = nvfp4_problem(None, 9, 128, 256, 1, rng)
        C = oracle.fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], p["alpha"])
    tot = brute_nvfp4(p["A"], p["B"], p["a_scale"], p["b_scale"], ids, p["alpha"])
    alpha = Fraction(float(p["alpha"]))
    for i in range(C.shape[0]):
        for n in range(C.shape[1]):
            exact = alpha * int(tot[i, n]) / (1 << 20)
            assert abs(C[i, n] - float(exact)) <= 2.0 ** -45 * (abs(float(exact)) + 1e-30) + 1e-300


def test_nvfp4_per_expert_alpha_equals_exact_integer():
    """Distinct per-expert alphas (not powers of two) against the exact
    integer brute force, expert by expert."""
    rng = np.random.default_rng(17)
    ids = np.array([2, 0, -1, 1, 2, 0, 0, 1], np.int32)
    p = nvfp4_problem(ids, 8, 128, 256, 3, rng)
    alphas = np.array([0.3, 1.75e-3, 37.0], np.float32)
    C = oracle.grouped_fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], ids, alphas)
    tot = brute_nvfp4(p["A"], p["B"], p["a_scale"], p["b_scale"], ids, None)
    for i in range(8):
        if ids[i] < 0:
            assert np.all(C[i] == 0.0)
            continue
        a = Fraction(float(alphas[ids[i]]))
        for n in range(128):
            exact = a * int(tot[i, n]) / (1 << 20)
            assert abs(C[i, n] - float(exact)) <= 2.0 ** -45 * (abs(float(exact)) + 1e-30) + 1e-300


def test_nvfp4_per_expert_alpha_invariants():
    rng = np.random.default_rng(18)
    ids = runs_to_indices([5, 0, 7, 4])
    p = nvfp4_problem(ids, ids.size, 128, 128, 4, rng)
    args = (p["A"], p["B"], p["a_scale"], p["b_scale"], ids)
    one = oracle.grouped_fp4_gemm(*args, np.float32(0.625))
    same = oracle.grouped_fp4_gemm(*args, np.full(4, 0.625, np.float32))
    assert np.array_equal(one, same)
    # scaling one expert's alpha by 2^k scales exactly that expert's rows
    base = oracle.grouped_fp4_gemm(*args, np.ones(4, np.float32))
    scaled = oracle.grouped_fp4_gemm(*args, np.array([1, 1, 8, 1], np.float32))
    assert np.array_equal(scaled[ids == 2], 8 * base[ids == 2])
    assert np.array_equal(scaled[ids != 2], base[ids != 2])


def test_nvfp4_problem_batch_slices_tile_one_problem():
    """Row slices and column slices of one dense problem, given as separate
    problems, tile that problem's result; problems of different K are each
    exact."""
    rng = np.random.default_rng(19)
    p = nvfp4_problem(None, 40, 384, 256, 1, rng)
    full = oracle.fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], p["alpha"])
    parts = [dict(A=p["A"][r], B=p["B"][c], a_scale=p["a_scale"][r], b_scale=p["b_scale"][c],
                  alpha=p["alpha"]) for r in (slice(0, 17), slice(17, 40))
             for c in (slice(0, 128), slice(128, 384))]
    out = oracle.fp4_gemm_problems(parts)
    assert np.array_equal(np.block([[out[0], out[1]], [out[2], out[3]]]), full)
    q = nvfp4_problem(None, 5, 128, 512, 1, np.random.default_rng(20))
    (c1, c2) = oracle.fp4_gemm_problems([p, q])
    tot = brute_nvfp4(q["A"], q["B"], q["a_scale"], q["b_scale"], None, None)
    exact = np.array([[float(Fraction(float(q["alpha"])) * int(t) / (1 << 20)) for t in row]
                      for row in tot])
    assert np.allclose(c2, exact, rtol=2.0 ** -45, atol=0) and c1.shape == (40, 384)


def test_w4a16_reproduces_w4a4_on_nvfp4_representable_activations():
    """Activations that are exactly NVFP4 values (qA sA gA) through the
    W4A16 form equal the W4A4 oracle with alpha = gA gB."""
    rng = np.random.default_rng(24)
    ids = np.array([1, -1, 0, 2, 2, 0, 1, 1, -1, 2], np.int32)
    p = nvfp4_problem(ids, 10, 256, 384, 3, rng)
    qa = _e2m1_values(p["A"])
    sa = oracle.decode_e4m3fn(p["a_scale"])
    ga = np.float32(0.375)
    A16 = (qa.reshape(10, 384 // 16, 16) * sa[:, :, None]).reshape(10, 384) * float(ga)
    gb = np.float32(p["alpha"])
    w4a16 = oracle.grouped_w4a16_gemm(A16, p["B"], p["b_scale"], ids, gb)
    w4a4 = oracle.grouped_fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], ids,
                                   np.float32(ga * gb))
    assert np.allclose(w4a16, w4a4, rtol=1e-12, atol=0)
    assert np.all(w4a16[ids == -1] == 0.0)


def _e2m1_values(packed):
    q = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    q[..., 0::2], q[..., 1::2] = packed & 0xF, packed >> 4
    return oracle.decode_e2m1(q)


def test_w4a16_equals_exact_rational():
    """BF16 activations (arbitrary 8-bit significands) against exact
    Fraction arithmetic, with a non-power-of-two global scale."""
    rng = np.random.default_rng(25)
    ids = np.array([0, 1, 1, -1, 0], np.int32)
    p = nvfp4_problem(ids, 5, 128, 128, 2, rng)
    A = rng.standard_normal((5, 128)).astype(np.float32)
    A = (A.view(np.uint32) & 0xFFFF0000).view(np.float32)  # BF16 values
    gb = np.float32(0.7)
    C = oracle.grouped_w4a16_gemm(A, p["B"], p["b_scale"], ids, gb)
    qb = _e2m1_values(p["B"])
    sb = oracle.decode_e4m3fn(p["b_scale"])
    for i in range(5):
        g = int(ids[i])
        for n in range(0, 128, 7):
            if g < 0:
                assert C[i, n] == 0.0
                continue
            terms = [Fraction(float(A[i, k])) * Fraction(float(qb[g, n, k]))
                     * Fraction(float(sb[g, n, k // 16])) * Fraction(float(gb))
                     for k in range(128)]
            exact, mag = sum(terms), float(sum(abs(t) for t in terms))
            assert abs(C[i, n] - float(exact)) <= 2.0 ** -45 * mag + 1e-300


# -------------------------------------------------------------- worked examples
@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_worked_examples(ex):
    d = build(ex)
    if d["kind"] == "fp8":
        C = oracle.grouped_fp8_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"])
    elif d["m_indices"] is None:
        C = oracle.fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["alpha"])
    else:
        C = oracle.grouped_fp4_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], d["m_indices"],
                                    d["alpha"])
    assert np.array_equal(C, d["expected"])
    assert np.array_equal(oracle.bf16_rne_bits(C), d["expected_bf16"])


# ------------------------------------------------------------------ invariants
def _small_fp8(seed=11, G=4):
    rng = np.random.default_rng(seed)
    ids = runs_to_indices([5, 0, 9, 3], pad_to=4)
    return fp8_problem(ids, 256, 256, G, rng), rng


def _fp8(p, **over):
    q = dict(p, **over)
    return oracle.grouped_fp8_gemm(q["A"], q["B"], q["a_scale"], q["b_scale"], q["m_indices"])


def test_inv_padding_rows_zero():
    p, _ = _small_fp8()
    C = _fp8(p)
    assert np.all(C[p["m_indices"] == -1] == 0.0)
    assert np.all(np.any(C[p["m_indices"] >= 0] != 0.0, axis=1))


def test_inv_expert_relabel():
    p, rng = _small_fp8()
    perm = rng.permutation(p["G"])  # expert g becomes perm[g]
    B2 = np.empty_like(p["B"])
    s2 = np.empty_like(p["b_scale"])
    B2[perm], s2[perm] = p["B"], p["b_scale"]
    ids2 = np.where(p["m_indices"] >= 0, perm[np.maximum(p["m_indices"], 0)], -1).astype(np.int32)
    assert np.array_equal(_fp8(p), _fp8(p, B=B2, b_scale=s2, m_indices=ids2))


def test_inv_row_permutation():
    p, rng = _small_fp8()
    perm = rng.permutation(p["M"])
    C = _fp8(p)
    C2 = _fp8(p, A=p["A"][perm], a_scale=p["a_scale"][perm], m_indices=p["m_indices"][perm])
    assert np.array_equal(C2, C[perm])


def test_inv_power_of_two_scales():
    p, _ = _small_fp8()
    C = _fp8(p)
    sa = p["a_scale"].copy()
    sa[3] *= np.float32(8.0)
    C2 = _fp8(p, a_scale=sa)
    assert np.array_equal(C2[3], 8.0 * C[3])
    assert np.array_equal(np.delete(C2, 3, axis=0), np.delete(C, 3, axis=0))
    sb = p["b_scale"].copy()
    sb[2, 1, :] *= np.float32(0.25)  # expert 2, columns 128..255
    C3 = _fp8(p, b_scale=sb)
    rows2 = p["m_indices"] == 2
    assert np.array_equal(C3[rows2, 128:], 0.25 * C[rows2, 128:])
    assert np.array_equal(C3[rows2, :128], C[rows2, :128])
    assert np.array_equal(C3[~rows2], C[~rows2])


def test_inv_sign_flip():
    p, _ = _small_fp8()
    assert np.array_equal(_fp8(p, A=p["A"] ^ np.uint8(0x80)), -_fp8(p))


def test_inv_zero_scales():
    p, _ = _small_fp8()
    assert np.all(_fp8(p, a_scale=np.zeros_like(p["a_scale"])) == 0.0)


def test_inv_grouped_fp4_single_expert_equals_dense():
    rng = np.random.default_rng(21)
    p = nvfp4_problem(np.zeros(12, np.int32), 12, 256, 512, 1, rng)
    Cg = oracle.grouped_fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], p["m_indices"],
                                 p["alpha"])
    Cd = oracle.fp4_gemm(p["A"], p["B"][0], p["a_scale"], p["b_scale"][0], p["alpha"])
    assert np.array_equal(Cg, Cd)


def test_rows_argument_selects_rows():
    p, _ = _small_fp8()
    rows = np.array([0, 7, 3, 16])
    full = _fp8(p)
    part = oracle.grouped_fp8_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], p["m_indices"],
                                   rows=rows)
    assert np.array_equal(part, full[rows])


# ------------------------------------------- reduction to a library routine
def test_unit_scales_single_expert_is_plain_matmul():
    rng = np.random.default_rng(5)
    ids = np.zeros(40, np.int32)
    p = fp8_problem(ids, 128, 512, 1, rng)
    ones_a = np.ones_like(p["a_scale"])
    ones_b = np.ones_like(p["b_scale"])
    C = oracle.grouped_fp8_gemm(p["A"], p["B"], ones_a, ones_b, ids)
    At = torch.from_numpy(p["A"]).view(torch.float8_e4m3fn).double()
    Bt = torch.from_numpy(p["B"][0]).view(torch.float8_e4m3fn).double()
    ref = (At @ Bt.T).numpy()
    assert np.array_equal(C, ref)  # every partial and total is exact in float64


def test_check_tolerance_rule():
    ref = np.array([[100.0, -1.0], [0.0, 0.0]])
    ids = np.array([0, -1])
    ok = oracle.check_tolerance(np.array([[100.9, -1.0], [0.0, 0.0]]), ref, ids)
    assert ok["ok"]
    bad = oracle.check_tolerance(np.array([[102.0, -1.0], [0.0, 0.0]]), ref, ids)
    assert not bad["ok"] and bad["n_bad"] == 1
    pad = oracle.check_tolerance(np.array([[100.0, -1.0], [0.0, 1e-9]]), ref, ids)
    assert not pad["ok"] and pad["n_pad_nonzero"] == 1
