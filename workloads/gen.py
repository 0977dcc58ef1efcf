"""Seeded workloads for the block-scaled (grouped) GEMM.

Every array comes from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed
draw order: expert row counts first, then A, then B.  The named configurations
are the MoE-shaped problems the kernels are measured and checked on:

  c1_tiny_fp8          FP8, G=2, M=256 (runs of 100 and 156: the expert
                       boundary falls inside the first 128-row window),
                       N=256, K=512, seed 0
  c2_moe_fp8           FP8, G=8, M=8192 rows in sorted contiguous runs with
                       counts ~ multinomial(8192, uniform), N=4096, K=7168
  c3_skewed_fp8        FP8, G=32, M=16384 incl. padding; Zipf(1.2) expert
                       counts, each run padded to a multiple of 128 with -1
                       rows, trailing -1 rows; A ~ Student-t(3); N=2048, K=7168
  c4_dense_nvfp4       NVFP4 dense, M=2048, N=36864, K=4608
  c5_moe_nvfp4         NVFP4 grouped, G=8 x 8192 rows, N=8192, K=8192
  p2_unaligned         FP8, M=65, N=128, K=128, G=2 (the flashinfer#7877
                       page's "correctness_unaligned_transition" shape)
  p2_m777_g8           FP8, M=777, N=256, K=512, G=8 (that page's
                       "random_s9_m777_g8_n256_k512" shape; seed 9)
  d5_decode_w4a16      W4A16 decode on c5's experts: 64 tokens x top-2 of
                       G=8 (128 rows, unsorted), BF16 activations, NVFP4
                       B [8, 8192, 8192], seed 0
  p4_problems_nvfp4    a batch of 8 dense NVFP4 problems of different
                       shapes for one launch (the cutlass#3124 page's
                       grouped GEMM over different M, N, K): expert g has
                       multinomial(16384, uniform) rows and alternately
                       (N, K) = (4096, 7168) and (7168, 2048), seed 0
  p8_problems_fp8      the same batch recipe with dense block-scaled FP8
                       problems (fp8_gemm_problems), seed 0

Padding rows (m_indices = -1) hold ordinary random data so that a kernel which
wrongly computes them is caught.
"""
from __future__ import annotations

import numpy as np

from .quant import quantize_fp8_blocks, quantize_fp8_rows, quantize_nvfp4, nvfp4_global_scale


def runs_to_indices(counts, pad_to: int = 1, total: int | None = None) -> np.ndarray:
    """Contiguous expert runs: expert g repeated counts[g] times, each run
    followed by -1 rows up to a multiple of ``pad_to``, then -1 rows up to
    ``total``."""
    parts = []
    for g, c in enumerate(counts):
        c = int(c)
        parts.append(np.full(c, g, dtype=np.int32))
        pad = (-c) % pad_to
        if pad:
            parts.append(np.full(pad, -1, dtype=np.int32))
    idx = np.concatenate(parts) if parts else np.zeros(0, np.int32)
    if total is not None:
        assert idx.size <= total
        idx = np.concatenate([idx, np.full(total - idx.size, -1, dtype=np.int32)])
    return idx.astype(np.int32)


def _draw(rng, dist: str, shape):
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "student_t3":
        return rng.standard_t(3, size=shape).astype(np.float32)
    raise ValueError(dist)


def fp8_problem(m_indices, N: int, K: int, G: int, rng, a_dist: str = "normal",
                b_dist: str = "normal") -> dict:
    """Quantised FP8 grouped-GEMM inputs for a given row routing."""
    m_indices = np.ascontiguousarray(m_indices, dtype=np.int32)
    M = m_indices.size
    X = _draw(rng, a_dist, (M, K))
    A, a_scale = quantize_fp8_rows(X)
    del X
    Bf = np.empty((G, N, K), np.float32)
    for g in range(G):
        Bf[g] = _draw(rng, b_dist, (N, K))
    B, b_scale = quantize_fp8_blocks(Bf.reshape(G * N, K))
    del Bf
    B = B.reshape(G, N, K)
    b_scale = b_scale.reshape(G, N // 128, K // 128)
    return dict(kind="fp8", A=A, B=B, a_scale=a_scale, b_scale=b_scale,
                m_indices=m_indices, M=M, N=N, K=K, G=G)


def nvfp4_problem(m_indices, M: int, N: int, K: int, G: int, rng) -> dict:
    """Quantised NVFP4 inputs.  ``m_indices`` None means dense (G = 1, no
    routing).  B shares one global scale over all experts."""
    X = _draw(rng, "normal", (M, K))
    A, a_sc, gA = quantize_nvfp4(X)
    del X
    Bf = np.empty((G, N, K), np.float32)
    for g in range(G):
        Bf[g] = _draw(rng, "normal", (N, K))
    gB = nvfp4_global_scale(float(np.abs(Bf).max()))
    B, b_sc, _ = quantize_nvfp4(Bf.reshape(G * N, K), gB)
    del Bf
    B = B.reshape(G, N, K // 2)
    b_sc = b_sc.reshape(G, N, K // 16)
    alpha = np.float32(np.float32(gA) * np.float32(gB))
    d = dict(kind="nvfp4", A=A, B=B, a_scale=a_sc, b_scale=b_sc, gA=gA, gB=gB,
             alpha=alpha, M=M, N=N, K=K, G=G)
    if m_indices is None:
        d["B"], d["b_scale"] = B[0], b_sc[0]
        d["m_indices"] = None
    else:
        d["m_indices"] = np.ascontiguousarray(m_indices, dtype=np.int32)
    return d


def w4a16_problem(m_indices, N: int, K: int, G: int, rng) -> dict:
    """BF16 activations (N(0,1) rounded to nearest even) routed by
    m_indices, and NVFP4 weights B [G, N, K/2] with one global scale."""
    m_indices = np.ascontiguousarray(m_indices, dtype=np.int32)
    M = m_indices.size
    X = _draw(rng, "normal", (M, K))
    u = X.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # RNE to BF16
    A = (bits.astype(np.uint32) << 16).view(np.float32)
    Bf = np.empty((G, N, K), np.float32)
    for g in range(G):
        Bf[g] = _draw(rng, "normal", (N, K))
    gB = nvfp4_global_scale(float(np.abs(Bf).max()))
    B, b_sc, _ = quantize_nvfp4(Bf.reshape(G * N, K), gB)
    del Bf
    return dict(kind="w4a16", A=A, A_bits=bits, B=B.reshape(G, N, K // 2),
                b_scale=b_sc.reshape(G, N, K // 16), b_global=np.float32(gB),
                m_indices=m_indices, M=M, N=N, K=K, G=G)


def decode_routing(tokens: int, top_k: int, G: int, rng) -> np.ndarray:
    """MoE decode routing: each token picks top_k distinct experts uniformly;
    row t * top_k + j of the expanded batch goes to token t's j-th expert
    (unsorted, as the router emits them)."""
    return np.stack([rng.choice(G, top_k, replace=False) for _ in range(tokens)]).reshape(-1) \
        .astype(np.int32)


def moe_expand(routing, G: int, pad_to: int = 1):
    """The row expansion of an MoE layer: routing [T, top_k] holds each
    token's experts; the expanded batch lists, expert by expert (tokens in
    order within an expert), one row per (token, expert) pair, each expert's
    run padded with padding rows to a multiple of pad_to.  Returns (rows,
    m_indices): rows[r] is the token of expanded row r (-1 for padding) and
    m_indices[r] its expert (-1 for padding)."""
    routing = np.asarray(routing)
    T = routing.shape[0]
    rows, ids = [], []
    for g in range(G):
        tok = np.nonzero((routing == g).any(axis=1))[0].astype(np.int32)
        pad = (-tok.size) % pad_to
        rows += [tok, np.full(pad, -1, np.int32)]
        ids += [np.full(tok.size, g, np.int32), np.full(pad, -1, np.int32)]
    assert T >= 1
    return np.concatenate(rows).astype(np.int32), np.concatenate(ids).astype(np.int32)


def bf16_activations(T: int, K: int, rng) -> tuple:
    """N(0,1) activations rounded to BF16 (nearest even): (float32 values,
    uint16 bit patterns)."""
    X = _draw(rng, "normal", (T, K))
    u = X.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32), bits


def _zipf_counts(rng, G=32, total_rows=16384, start_T=14336, s=1.2, pad_to=128):
    p = (np.arange(1, G + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    T = start_T
    while True:
        counts = rng.multinomial(T, p)
        padded = int(sum(int(c) + ((-int(c)) % pad_to) for c in counts))
        if padded <= total_rows:
            return counts
        T -= pad_to


def make(name: str, seed: int | None = None) -> dict:
    """Build a named workload (see the module docstring)."""
    if name == "c1_tiny_fp8":
        rng = np.random.default_rng(0 if seed is None else seed)
        idx = runs_to_indices([100, 156])
        return fp8_problem(idx, 256, 512, 2, rng)
    if name == "c2_moe_fp8":
        rng = np.random.default_rng(0 if seed is None else seed)
        counts = rng.multinomial(8192, [1 / 8] * 8)
        return fp8_problem(runs_to_indices(counts), 4096, 7168, 8, rng)
    if name == "c3_skewed_fp8":
        rng = np.random.default_rng(0 if seed is None else seed)
        counts = _zipf_counts(rng)
        idx = runs_to_indices(counts, pad_to=128, total=16384)
        return fp8_problem(idx, 2048, 7168, 32, rng, a_dist="student_t3")
    if name == "c4_dense_nvfp4":
        rng = np.random.default_rng(0 if seed is None else seed)
        return nvfp4_problem(None, 2048, 36864, 4608, 1, rng)
    if name == "c5_moe_nvfp4":
        rng = np.random.default_rng(0 if seed is None else seed)
        idx = np.repeat(np.arange(8, dtype=np.int32), 8192)
        return nvfp4_problem(idx, 65536, 8192, 8192, 8, rng)
    if name == "p2_unaligned":
        rng = np.random.default_rng(9 if seed is None else seed)
        counts = rng.multinomial(65, [1 / 2] * 2)
        return fp8_problem(runs_to_indices(counts), 128, 128, 2, rng)
    if name == "p2_m777_g8":
        rng = np.random.default_rng(9 if seed is None else seed)
        counts = rng.multinomial(777, [1 / 8] * 8)
        return fp8_problem(runs_to_indices(counts), 256, 512, 8, rng)
    if name == "d5_decode_w4a16":
        rng = np.random.default_rng(0 if seed is None else seed)
        idx = decode_routing(64, 2, 8, rng)
        return w4a16_problem(idx, 8192, 8192, 8, rng)
    if name == "p4_problems_nvfp4":
        rng = np.random.default_rng(0 if seed is None else seed)
        counts = rng.multinomial(16384, [1 / 8] * 8)
        probs = []
        for g, m in enumerate(counts):
            N, K = (4096, 7168) if g % 2 == 0 else (7168, 2048)
            probs.append(nvfp4_problem(None, int(m), N, K, 1, rng))
        return dict(kind="fp4_problems", problems=probs, G=len(probs))
    if name == "p8_problems_fp8":
        rng = np.random.default_rng(0 if seed is None else seed)
        counts = rng.multinomial(16384, [1 / 8] * 8)
        probs = []
        for g, m in enumerate(counts):
            N, K = (4096, 7168) if g % 2 == 0 else (7168, 2048)
            probs.append(fp8_problem(np.zeros(int(m), np.int32), N, K, 1, rng))
        return dict(kind="fp8_problems", problems=probs, G=len(probs))
    raise KeyError(name)


def real_rows(problem: dict) -> int:
    if problem["kind"] in ("fp4_problems", "fp8_problems"):
        return sum(q["M"] for q in problem["problems"])
    idx = problem.get("m_indices")
    if idx is None:
        return problem["M"]
    G = problem["G"]
    return int(np.count_nonzero((idx >= 0) & (idx < G)))


CONFIGS = ("c1_tiny_fp8", "c2_moe_fp8", "c3_skewed_fp8", "c4_dense_nvfp4", "c5_moe_nvfp4",
           "p2_unaligned", "p2_m777_g8")
