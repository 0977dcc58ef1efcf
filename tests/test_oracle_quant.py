"""Pins of the activation-quantiser oracle (oracle/quant.py) against the
format definitions, exhaustive enumeration, a library cast and exact
reconstruction.  CPU only."""
import numpy as np
import pytest

from oracle import decode_e2m1, decode_e4m3fn
from oracle.quant import (e2m1_round, e4m3fn_round, nvfp4_global_scale, quantize_fp8_1x128,
                          quantize_nvfp4)

FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def test_e4m3_every_finite_code_round_trips():
    v = decode_e4m3fn(FINITE_E4M3).astype(np.float32)
    assert np.array_equal(e4m3fn_round(v), FINITE_E4M3)


def test_e4m3_midpoints_round_to_even_and_neighbours_to_nearest():
    codes = np.arange(0x7F, dtype=np.uint8)
    v = decode_e4m3fn(codes)
    lo, hi = v[:-1], v[1:]
    mid = ((lo + hi) / 2).astype(np.float32)  # 5 significant bits: exact in FP32
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(e4m3fn_round(mid), even)
    assert np.array_equal(e4m3fn_round(-mid), even | 0x80)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(e4m3fn_round(below), codes[:-1])
    assert np.array_equal(e4m3fn_round(above), codes[1:])


def test_e4m3_round_matches_torch_cast_of_clamped_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(40),
        rng.uniform(-448, 448, 20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-3).astype(np.float32),
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -9 * 1.5], np.float32),
    ])
    ours = e4m3fn_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e2m1_round_trip_and_midpoints():
    codes = np.arange(16, dtype=np.uint8)
    v = decode_e2m1(codes).astype(np.float32)
    back = e2m1_round(v)
    assert np.array_equal(back[codes != 8], codes[codes != 8])  # -0 keeps its sign: code 8
    assert back[8] == 8
    pos = np.arange(8, dtype=np.uint8)
    pv = decode_e2m1(pos)
    mid = ((pv[:-1] + pv[1:]) / 2).astype(np.float32)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(e2m1_round(mid), even)  # e.g. 5 -> 4 (code 6), 2.5 -> 2 (code 4)
    assert e2m1_round(np.float32(5.0)) == 6 and e2m1_round(np.float32(2.5)) == 4


def _nearest_brute(y, table_codes):
    """Brute force: nearest code over the whole table, ties to the even
    code, sign from the input."""
    vals = np.abs(table_codes[1])
    a = np.abs(y.astype(np.float64))[:, None]
    d = np.abs(a - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    code = np.where(cand & (table_codes[0][None, :] % 2 == 0), table_codes[0][None, :], 255)
    first = np.where(cand.sum(axis=1) > 1, code.min(axis=1), table_codes[0][d.argmin(axis=1)])
    return first.astype(np.uint8)


def test_fp8_1x128_codes_are_nearest_and_scales_exact():
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((6, 512)) * np.exp(rng.uniform(-6, 6, (6, 1)))).astype(np.float32)
    X[2, 128:256] = 0.0  # an all-zero block
    codes, scale = quantize_fp8_1x128(X)
    amax = np.abs(X.reshape(6, 4, 128)).max(axis=2)
    assert np.array_equal(scale, np.where(amax > 0, amax / np.float32(448), np.float32(1)))
    assert scale[2, 1] == 1.0 and not codes[2, 128:256].any()
    y = np.clip((X.reshape(6, 4, 128) / scale[:, :, None]).astype(np.float32), -448, 448).reshape(-1)
    tc = np.arange(0x7F, dtype=np.uint8)
    brute = _nearest_brute(y, (tc, decode_e4m3fn(tc)))
    assert np.array_equal(codes.reshape(-1) & 0x7F, brute)
    assert np.array_equal(codes.reshape(-1) >> 7, np.signbit(y).astype(np.uint8))


def test_fp8_1x128_reconstructs_inputs_built_from_codes():
    """Blocks whose largest element is code 0x7E (448) times a scale s give
    back exactly s and the codes (every FP32 step is exact: x / s is a code
    value because s = 448 s / 448 and x = value * s with a power-of-two s)."""
    rng = np.random.default_rng(6)
    M, K = 8, 384
    codes = rng.choice(FINITE_E4M3[FINITE_E4M3 != 0x80], (M, K)).astype(np.uint8)
    codes[:, ::128] = 0x7E  # amax of each block is 448 * s
    s = np.exp2(rng.integers(-20, 10, (M, K // 128))).astype(np.float32)
    X = (decode_e4m3fn(codes).reshape(M, K // 128, 128) * s[:, :, None]).reshape(M, K)
    X = X.astype(np.float32)
    got, scale = quantize_fp8_1x128(X)
    assert np.array_equal(scale, s)
    assert np.array_equal(got, codes)


def test_nvfp4_global_scale_and_zero():
    X = np.array([[0.0, 3.0, -8064.0, 1.0] * 4], np.float32)
    assert nvfp4_global_scale(X) == np.float32(8064.0) / np.float32(2688.0) == np.float32(3.0)
    assert nvfp4_global_scale(np.zeros((2, 16), np.float32)) == 1.0


def test_nvfp4_reconstructs_inputs_built_from_codes():
    """With a power-of-two global scale and each block's largest element code
    7 (6.0), x / (s g) recovers every code and s recovers each scale code."""
    rng = np.random.default_rng(7)
    M, K = 6, 256
    g = np.float32(2.0 ** -7)
    q = rng.integers(0, 16, (M, K)).astype(np.uint8)
    q[q == 8] = 0  # -0 would come back as +0 from 0 * s
    q[:, ::16] = 7
    sc = rng.choice(FINITE_E4M3[(FINITE_E4M3 < 0x78) & (FINITE_E4M3 > 0x07)], (M, K // 16))
    val = decode_e2m1(q).reshape(M, K // 16, 16) * decode_e4m3fn(sc)[:, :, None] * float(g)
    X = val.reshape(M, K).astype(np.float32)
    assert np.array_equal(X.astype(np.float64), val.reshape(M, K))  # exact in FP32
    packed, s_code, g_out = quantize_nvfp4(X, g)
    assert g_out == g
    assert np.array_equal(s_code, sc)
    unpacked = np.empty((M, K), np.uint8)
    unpacked[:, 0::2] = packed & 0xF
    unpacked[:, 1::2] = packed >> 4
    assert np.array_equal(unpacked, q)


def test_nvfp4_codes_are_nearest_given_the_block_scale():
    rng = np.random.default_rng(8)
    X = (rng.standard_normal((5, 128)) * 3).astype(np.float32)
    X[1, 16:32] = 0.0
    packed, s_code, g = quantize_nvfp4(X)
    assert g == np.float32(np.abs(X).max()) / np.float32(2688)
    Xb = X.reshape(5, 8, 16)
    bamax = np.abs(Xb).max(axis=2)
    assert np.array_equal(s_code, e4m3fn_round(np.minimum((bamax / (np.float32(6) * g)).astype(
        np.float32), np.float32(448))))
    assert s_code[1, 1] == 0
    d = (decode_e4m3fn(s_code).astype(np.float32) * g).astype(np.float32)
    q = np.empty((5, 128), np.uint8)
    q[:, 0::2] = packed & 0xF
    q[:, 1::2] = packed >> 4
    assert not q[1, 16:32].any()
    y = np.clip((Xb / np.where(d > 0, d, 1)[:, :, None]).astype(np.float32), -6, 6).reshape(-1)
    tc = np.arange(8, dtype=np.uint8)
    brute = _nearest_brute(y, (tc, decode_e2m1(tc)))
    keep = np.repeat(d.reshape(-1) > 0, 16)
    assert np.array_equal((q.reshape(-1) & 7)[keep], brute[keep])
    assert np.array_equal((q.reshape(-1) >> 3)[keep], np.signbit(y).astype(np.uint8)[keep])
