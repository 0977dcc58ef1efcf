"""Pins of the oracle's format decoders and of the input quantisers.

Each decoder is compared with something other than itself: an exhaustive
integer re-derivation of every code, PyTorch's own float8_e4m3fn / bfloat16
conversions (an independent implementation), and the constants the pages
print (E4M3FN's largest finite value 448, sglang#27745 page, "Code analysis
1: FP8 quantisation")."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import quant


def _e4m3_fraction(code: int):
    """Independent decode: value = (integer significand) * 2^-9 * 2^shift."""
    s = -1 if code & 0x80 else 1
    E, M = (code >> 3) & 15, code & 7
    if E == 15 and M == 7:
        return None
    sig = M if E == 0 else (8 + M) << (E - 1)
    return s * Fraction(sig, 512)


def test_e4m3_exhaustive_against_integer_form():
    v = oracle.decode_e4m3fn(np.arange(256))
    for c in range(256):
        f = _e4m3_fraction(c)
        if f is None:
            assert math.isnan(v[c]), hex(c)
        else:
            assert Fraction(float(v[c])) == f, hex(c)


def test_e4m3_exhaustive_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = oracle.decode_e4m3fn(np.arange(256))
    nan = np.isnan(tv)
    assert np.array_equal(nan, np.isnan(ov))
    assert np.array_equal(tv[~nan], ov[~nan])


def test_e4m3_printed_constants():
    d = oracle.decode_e4m3fn
    assert d(0x7E) == 448.0  # largest finite E4M3FN value on gfx950
    assert np.nanmax(d(np.arange(256))) == 448.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x01) == 2.0 ** -9 and d(0x08) == 2.0 ** -6 and d(0x38) == 1.0
    assert d(0x80) == 0.0 and d(0xB8) == -1.0
    assert not np.isinf(d(np.arange(256))).any()  # no infinities in the FN variant


def test_e2m1_exhaustive():
    v = oracle.decode_e2m1(np.arange(16))
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(v[:8]) == table
    assert list(v[8:]) == [-t for t in table]


def test_unpack_low_nibble_first():
    p = np.array([[0x21, 0x7F]], np.uint8)
    assert oracle.unpack_e2m1(p).tolist() == [[0x1, 0x2, 0xF, 0x7]]


def test_bf16_rne_against_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * 1e3,
                        rng.standard_normal(1000) * 1e-30,
                        # exact ties: 8 significant bits + a half ulp
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 256 + 1, 256 + 3,
                                  0.0, -0.0, 3.0e38])]).astype(np.float32)
    ob = oracle.bf16_rne_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ob, tb)
    back = oracle.bf16_bits_to_float(ob)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_quantiser_e4m3_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(300000) * 60, np.linspace(-460, 460, 100001),
                        np.array([2 ** -10, 3 * 2 ** -10, 448.0, 449.0, -2 ** -11])]).astype(np.float32)
    c = quant.e4m3fn_encode(x)
    t = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c, t)


def test_quantiser_e2m1_is_nearest_even():
    y = np.linspace(-7, 7, 28001).astype(np.float32)
    e = quant.e2m1_encode(y)
    dec = oracle.decode_e2m1(e)
    a = np.minimum(np.abs(y.astype(np.float64)), 6.0)
    mags = oracle.decode_e2m1(np.arange(8))
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1)
    assert np.array_equal(np.abs(dec) - a, np.abs(dec) - a)  # finite
    assert np.all(np.abs(np.abs(dec) - a) == best)  # nearest
    ties = (dist == best[:, None]).sum(axis=1) == 2
    assert np.all((e[ties] & 1) == 0)  # ties to even significand


@pytest.mark.parametrize("shape", [(3, 256), (128, 384)])
def test_quantiser_fp8_roundtrip(shape):
    rng = np.random.default_rng(5)
    X = rng.standard_normal(shape).astype(np.float32)
    codes, scale = quant.quantize_fp8_rows(X)
    deq = oracle.decode_e4m3fn(codes) * np.repeat(scale.astype(np.float64), 128, axis=1)
    # E4M3 keeps 4 significant bits: relative error <= 2^-4 for normal values
    err = np.abs(deq - X)
    assert np.all(err <= 2.0 ** -4 * np.abs(X) + 2.0 ** -9 * np.repeat(scale, 128, axis=1))
    assert np.all(np.abs(oracle.decode_e4m3fn(codes)) <= 448)


def test_quantiser_nvfp4_roundtrip():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((64, 256)).astype(np.float32)
    packed, sc, g = quant.quantize_nvfp4(X)
    q = oracle.decode_e2m1(oracle.unpack_e2m1(packed))
    s = np.repeat(oracle.decode_e4m3fn(sc), 16, axis=1)
    deq = q * s * float(g)
    # E2M1 keeps 2 significant bits: a half-step is at most 1/4 relative (1/3 at 1.5),
    # plus the saturating block max; check the block-relative error
    bmax = np.repeat(np.abs(X).reshape(64, 16, 16).max(axis=2), 16, axis=1)
    assert np.all(np.abs(deq - X) <= 0.26 * bmax + 1e-6)
    assert np.all(np.abs(q) <= 6)
