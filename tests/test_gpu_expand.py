"""The activation quantisers fused with the MoE row expansion, on the GPU
through the C ABI (quantize_fp8_1x128_rows, quantize_nvfp4_static_rows; the
onnxruntime#29824 page, "Code analysis 1": expandInputRowsKernel quantises
while it copies each token to the rows of its experts).

Codes and scales must equal the oracle's quantisation of the expanded rows
X[rows] bit for bit (padding rows: the encoding of a zero row), and the
grouped GEMM on them must match the oracle GEMM on the oracle-quantised
operand to the usual tolerance."""
import numpy as np
import pytest

import oracle
import oracle.quant as oq
import fp4_grouped_gemm_amd as fgg
from tests.gpu_util import c_to_f64, log
from workloads import bf16_activations, decode_routing, fp8_problem, moe_expand, nvfp4_problem

pytestmark = pytest.mark.gpu


def _expanded(X, rows):
    Xg = np.zeros((rows.size, X.shape[1]), np.float32)
    ok = (rows >= 0) & (rows < X.shape[0])
    Xg[ok] = X[rows[ok]]
    return Xg


def _setup(T, K, G, top_k, pad_to, seed):
    rng = np.random.default_rng(seed)
    routing = decode_routing(T, top_k, G, rng).reshape(T, top_k)
    rows, ids = moe_expand(routing, G, pad_to)
    X, bits = bf16_activations(T, K, rng)
    return rng, rows, ids, X, bits


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("T,K,G,top_k,pad_to,seed", [(300, 512, 5, 2, 16, 1),
                                                     (97, 384, 3, 1, 128, 2),
                                                     (64, 7168, 8, 2, 1, 3)])
def test_fp8_expand_bitwise_and_gemm(T, K, G, top_k, pad_to, seed):
    import torch
    rng, rows, ids, X, bits = _setup(T, K, G, top_k, pad_to, seed)
    Xd = _dev(bits.view(np.int16)).view(torch.bfloat16)
    log(f"fp8 expand T={T} K={K} G={G} R={rows.size}")
    Q, S = fgg.quantize_fp8_1x128(Xd, rows=_dev(rows))
    q_ref, s_ref = oq.quantize_fp8_1x128(_expanded(X, rows))
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    assert np.array_equal(S.cpu().numpy(), s_ref)
    # the grouped GEMM on the expanded operand
    p = fp8_problem(ids, 256, K, G, rng)
    log("fp8 expand -> grouped_fp8_gemm")
    C = fgg.grouped_fp8_gemm(Q, _dev(p["B"]), S, _dev(p["b_scale"]), _dev(ids))
    ref = oracle.grouped_fp8_gemm(q_ref, p["B"], s_ref, p["b_scale"], ids)
    res = oracle.check_tolerance(c_to_f64(C), ref, ids)
    assert res["ok"], res


@pytest.mark.parametrize("T,K,G,top_k,pad_to,seed", [(300, 512, 5, 2, 16, 4),
                                                     (50, 640, 4, 2, 128, 5)])
def test_nvfp4_static_expand_bitwise_and_gemm(T, K, G, top_k, pad_to, seed):
    import torch
    rng, rows, ids, X, bits = _setup(T, K, G, top_k, pad_to, seed)
    g = float(oq.nvfp4_global_scale(X))
    Xd = _dev(bits.view(np.int16)).view(torch.bfloat16)
    log(f"nvfp4 expand T={T} K={K} G={G} R={rows.size}")
    Q, S, _ = fgg.quantize_nvfp4(Xd, global_scale=g, rows=_dev(rows))
    q_ref, s_ref, _ = oq.quantize_nvfp4(_expanded(X, rows), np.float32(g))
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    assert np.array_equal(S.cpu().numpy(), s_ref)
    p = nvfp4_problem(ids, ids.size, 256, K, G, rng)
    alpha = float(np.float32(g) * np.float32(p["gB"]))
    log("nvfp4 expand -> grouped_fp4_gemm")
    C = fgg.grouped_fp4_gemm(Q, _dev(p["B"]), S, _dev(p["b_scale"]), _dev(ids), alpha)
    ref = oracle.grouped_fp4_gemm(q_ref, p["B"], s_ref, p["b_scale"], ids, alpha)
    res = oracle.check_tolerance(c_to_f64(C), ref, ids)
    assert res["ok"], res


def test_expand_out_of_range_rows_are_zero_rows():
    """Entries outside [0, T) -- -1, T, a large value -- encode zero rows
    (FP8: codes 0, scale 1.0; NVFP4: codes 0, scale code 0)."""
    import torch
    T, K = 40, 256
    rng = np.random.default_rng(6)
    X, bits = bf16_activations(T, K, rng)
    rows = np.array([3, -1, T, 7, 1 << 30, -5, 39, 0], np.int32)
    Xd = _dev(bits.view(np.int16)).view(torch.bfloat16)
    log("expand with out-of-range rows")
    Q, S = fgg.quantize_fp8_1x128(Xd, rows=_dev(rows))
    q_ref, s_ref = oq.quantize_fp8_1x128(_expanded(X, rows))
    assert np.array_equal(Q.cpu().numpy(), q_ref) and np.array_equal(S.cpu().numpy(), s_ref)
    bad = (rows < 0) | (rows >= T)
    assert np.all(Q.cpu().numpy()[bad] == 0) and np.all(S.cpu().numpy()[bad] == 1.0)
    g = float(oq.nvfp4_global_scale(X))
    Q4, S4, _ = fgg.quantize_nvfp4(Xd, global_scale=g, rows=_dev(rows))
    assert np.all(Q4.cpu().numpy()[bad] == 0) and np.all(S4.cpu().numpy()[bad] == 0)


def test_expand_graph_replay_rereads_rows():
    """rows is read on the device at every launch: a captured expansion
    replayed after the routing changes gives the new routing's rows."""
    import torch
    T, K = 80, 256
    rng = np.random.default_rng(7)
    X, bits = bf16_activations(T, K, rng)
    Xd = _dev(bits.view(np.int16)).view(torch.bfloat16)
    rows = rng.permutation(T).astype(np.int32)
    rd = _dev(rows)
    Q = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    S = torch.empty((T, K // 128), dtype=torch.float32, device="cuda")
    lib = fgg.load_library()

    def call():
        st = lib.quantize_fp8_1x128_rows(Xd.data_ptr(), rd.data_ptr(), Q.data_ptr(), S.data_ptr(),
                                         T, T, K, torch.cuda.current_stream().cuda_stream)
        assert st == 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("expand graph capture")
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        new = rng.permutation(T).astype(np.int32)
        new[rep] = -1
        rd.copy_(torch.from_numpy(new))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        q_ref, s_ref = oq.quantize_fp8_1x128(_expanded(X, new))
        assert np.array_equal(Q.cpu().numpy(), q_ref) and np.array_equal(S.cpu().numpy(), s_ref)
