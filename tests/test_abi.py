"""The C ABI on the host: the library loads, exports every function that
include/fgg.h declares, rejects bad arguments before touching a device, and
ranks tile configs.  No test here launches a kernel."""
import ctypes
import os
import re

import pytest

import fp4_grouped_gemm_amd as fgg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fgg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("grouped_fp8_gemm", "fp4_gemm", "grouped_fp4_gemm", "fgg_last_error"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(fgg.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing


def test_status_values():
    """The status codes of the C ABI, by name and number, as the header
    defines them (the binding's named-check convention of the flashinfer#7877
    page, "Code analysis 1", with one status per kind of failure)."""
    src = open(os.path.join(ROOT, "include", "fgg.h")).read()
    body = src[src.index("typedef enum {"):src.index("} fgg_status;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    vals = dict((k, int(v)) for k, v in re.findall(r"(FGG_\w+)\s*=\s*(\d+)", body))
    assert vals == {"FGG_OK": 0, "FGG_EINVAL": 1, "FGG_EUNSUPPORTED": 2, "FGG_EALIGN": 3,
                    "FGG_EDEVICE": 4, "FGG_EHIP": 5}
    assert (fgg.OK, fgg.EINVAL, fgg.EUNSUPPORTED, fgg.EALIGN, fgg.EDEVICE, fgg.EHIP) == \
        (0, 1, 2, 3, 4, 5)


P = 0x10000  # a 16-byte aligned non-null address; never dereferenced: each
# call below fails validation before anything touches a device.


def _fp8(A=P, B=P, sa=P, sb=P, mi=P, C=P, M=256, N=256, K=512, G=2):
    lib = fgg.load_library()
    st = lib.grouped_fp8_gemm(A, B, sa, sb, mi, C, M, N, K, G, None)
    return st, lib.fgg_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(A=0), 1, "null"),
    (dict(mi=0), 1, "m_indices"),
    (dict(M=0), 1, "M"),
    (dict(M=(1 << 24) + 1), 1, "M"),
    (dict(N=32), 1, "64 <= N"),
    (dict(N=200), 1, "N % 64"),
    (dict(N=64), 2, "N % 128"),
    (dict(N=192), 2, "N % 128"),
    (dict(K=200), 1, "K % 128"),
    (dict(K=64), 1, "K"),
    (dict(G=0), 1, "G"),
    (dict(A=P + 8), 3, "aligned"),
    (dict(C=P + 2), 3, "aligned"),
    (dict(sa=P + 2), 3, "aligned"),
])
def test_fp8_validation(kw, status, needle):
    st, msg = _fp8(**kw)
    assert st == status
    assert msg.startswith("grouped_fp8_gemm:") and needle in msg


def test_fp4_validation():
    lib = fgg.load_library()
    st = lib.fp4_gemm(P, P, P, P, 1.0, P, 100, 256, 144, None)
    assert st == 2 and "K % 128" in lib.fgg_last_error().decode()
    st = lib.fp4_gemm(P, P, P, P, 1.0, P, 100, 256, 136, None)
    assert st == 1 and "K % 16" in lib.fgg_last_error().decode()
    st = lib.fp4_gemm(P, P, P, P, float("inf"), P, 100, 256, 128, None)
    assert st == 1 and "alpha" in lib.fgg_last_error().decode()
    st = lib.grouped_fp4_gemm(P, P, P, P, 0, 1.0, P, 100, 256, 128, 2, None)
    assert st == 1 and "m_indices" in lib.fgg_last_error().decode()
    st = lib.grouped_fp4_gemm(P, P, P + 4, P, P, 1.0, P, 100, 256, 128, 2, None)
    assert st == 3


def test_quantizer_validation():
    lib = fgg.load_library()
    st = lib.quantize_fp8_1x128(P, P, P, 8, 200, None)
    assert st == 1 and lib.fgg_last_error().decode().startswith("quantize_fp8_1x128:")
    assert lib.quantize_fp8_1x128(0, P, P, 8, 256, None) == 1
    assert lib.quantize_fp8_1x128(P, P, P + 2, 8, 256, None) == 3
    assert lib.quantize_fp8_1x128(P + 4, P, P, 8, 256, None) == 3
    assert lib.quantize_fp8_1x128(P, P, P, 0, 256, None) == 1
    st = lib.quantize_nvfp4(P, P, P, 0, 8, 256, None)
    assert st == 1 and "global_scale" in lib.fgg_last_error().decode()
    assert lib.quantize_nvfp4(P, P, P, P + 2, 8, 256, None) == 3
    assert lib.quantize_nvfp4(P, P + 8, P, P, 8, 256, None) == 3
    assert lib.quantize_nvfp4_static(P, P, P, 1.0, 8, 200, None) == 1
    assert lib.quantize_nvfp4_static(P, P, P, 1.0, 8, 144, None) == 2
    assert lib.quantize_nvfp4_static(P, P + 8, P, 1.0, 8, 256, None) == 3
    for g in (0.0, -1.0, float("nan"), float("inf"), 1e-40):
        st = lib.quantize_nvfp4_static(P, P, P, g, 8, 256, None)
        assert st == 1 and "global_scale" in lib.fgg_last_error().decode()


def test_tune_validation_and_cache_without_gpu():
    """The *_tune entry points check their GEMM's arguments first (same
    messages, named after the tune call); with no tuning recorded the cache
    answers -1, and clearing it is always allowed."""
    lib = fgg.load_library()
    rep = fgg._TuneReport()
    st = lib.grouped_fp8_gemm_tune(P, P, P, P, P, P, 256, 256, 200, 2, 4, 5, ctypes.byref(rep),
                                   None, None)
    msg = lib.fgg_last_error().decode()
    assert st == 1 and msg.startswith("grouped_fp8_gemm_tune:") and "K % 128" in msg
    st = lib.fp4_gemm_tune(P, P, P, P, float("nan"), P, 100, 256, 128, 4, 5, None, None, None)
    assert st == 1 and "alpha" in lib.fgg_last_error().decode()
    st = lib.grouped_fp4_gemm_tune(P, P, P, P, 0, 1.0, P, 100, 256, 128, 2, 4, 5, None, None,
                                   None)
    assert st == 1 and lib.fgg_last_error().decode().startswith("grouped_fp4_gemm_tune:")
    # the tuning chooses the tile: an explicit one is an error (before any device call)
    opt = fgg._Options(0, 0, 0, 128)
    st = lib.grouped_fp8_gemm_tune(P, P, P, P, P, P, 256, 256, 512, 2, 4, 5, None,
                                   ctypes.byref(opt), None)
    assert st == 1 and "tile_id" in lib.fgg_last_error().decode()
    opt = fgg._Options(-1, 0, 0, -4)
    st = lib.grouped_fp4_gemm_tune(P, P, P, P, P, 1.0, P, 100, 256, 128, 2, 4, 5, None,
                                   ctypes.byref(opt), None)
    assert st == 1 and "run_align" in lib.fgg_last_error().decode()
    assert lib.fgg_tuned_tile(fgg.FP8, 256, 256, 512, 2) == -1
    lib.fgg_tune_clear()
    assert fgg.tuned_tile(fgg.FP4, 2048, 36864, 4608) == -1


def test_problem_batch_and_expert_alpha_validation():
    lib = fgg.load_library()
    arr = (fgg._Fp4Problem * 3)()
    for g in range(3):
        arr[g] = fgg._Fp4Problem(P, P, P, P, P, 100, 256, 512, 1.0)
    assert lib.fp4_gemm_problems(arr, 0, None) == 1
    assert "count" in lib.fgg_last_error().decode()
    assert lib.fp4_gemm_problems(arr, fgg.MAX_PROBLEMS + 1, None) == 1
    arr[1].K = 200
    st = lib.fp4_gemm_problems(arr, 3, None)
    msg = lib.fgg_last_error().decode()
    assert st == 1 and "problem 1" in msg and "K % 16" in msg
    arr[1].K = 512
    arr[2].alpha = float("inf")
    st = lib.fp4_gemm_problems(arr, 3, None)
    assert st == 1 and "problem 2" in lib.fgg_last_error().decode()
    arr[2].alpha = 1.0
    arr[0].C = P + 4
    assert lib.fp4_gemm_problems(arr, 3, None) == 3
    st = lib.grouped_fp4_gemm_alpha(P, P, P, P, P, 0, P, 100, 256, 128, 2, None)
    assert st == 1 and "alpha" in lib.fgg_last_error().decode()
    assert lib.grouped_fp4_gemm_alpha(P, P, P, P, P, P + 2, P, 100, 256, 128, 2, None) == 3
    st = lib.grouped_fp4_gemm_alpha(P, P, P, P, P, P, P, 100, 256, 100, 2, None)
    assert st == 1 and lib.fgg_last_error().decode().startswith("grouped_fp4_gemm_alpha:")


def test_fp8_problem_batch_validation():
    lib = fgg.load_library()
    arr = (fgg._Fp8Problem * 3)()
    for g in range(3):
        arr[g] = fgg._Fp8Problem(P, P, P, P, P, 100, 256, 512)
    assert lib.fp8_gemm_problems(arr, 0, None) == 1
    assert "count" in lib.fgg_last_error().decode()
    assert lib.fp8_gemm_problems(arr, fgg.MAX_PROBLEMS + 1, None) == 1
    arr[1].K = 200
    st = lib.fp8_gemm_problems(arr, 3, None)
    msg = lib.fgg_last_error().decode()
    assert st == 1 and "problem 1" in msg and "K % 128" in msg
    arr[1].K = 512
    arr[2].N = 192
    st = lib.fp8_gemm_problems(arr, 3, None)
    msg = lib.fgg_last_error().decode()
    assert st == 2 and "problem 2" in msg  # N % 128 != 0: unsupported
    arr[2].N = 256
    arr[0].b_scale = P + 2
    assert lib.fp8_gemm_problems(arr, 3, None) == 3
    assert lib.fgg_last_error().decode().startswith("fp8_gemm_problems (problem 0):")


def test_w4a16_validation():
    lib = fgg.load_library()
    st = lib.grouped_w4a16_gemm(P, P, P, P, 1.0, P, 16, 256, 200, 2, None)
    msg = lib.fgg_last_error().decode()
    assert st == 1 and msg.startswith("grouped_w4a16_gemm:") and "K % 16" in msg
    st = lib.grouped_w4a16_gemm(P, P, P, P, 1.0, P, 16, 256, 208, 2, None)
    assert st == 2 and "K % 128" in lib.fgg_last_error().decode()
    assert lib.grouped_w4a16_gemm(P, P, P, 0, 1.0, P, 16, 256, 256, 2, None) == 1
    assert lib.grouped_w4a16_gemm(P + 8, P, P, P, 1.0, P, 16, 256, 256, 2, None) == 3
    st = lib.grouped_w4a16_gemm(P, P, P, P, 1.0, P, 1 << 20, 256, 1024, 2, None)
    assert st == 2 and "2^31" in lib.fgg_last_error().decode()
    st = lib.grouped_w4a16_gemm(P, P, P, P, float("nan"), P, 16, 256, 256, 2, None)
    assert st == 1 and "b_global" in lib.fgg_last_error().decode()


def test_python_binding_raises_value_error():
    torch = pytest.importorskip("torch")
    A = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        fgg.grouped_fp8_gemm(A, torch.zeros((1, 128, 128), dtype=torch.uint8),
                             torch.ones((4, 1)), torch.ones((1, 1, 1)),
                             torch.zeros(4, dtype=torch.int32))  # CPU tensors


def test_ranker_orders_and_scores():
    for kind in (fgg.FP8, fgg.FP4):
        r = fgg.rank_tiles(kind, 8192, 4096, 7168, 8, num_cus=256)
        assert len(r) == fgg.num_tiles(kind) >= 1
        scores = [t["score"] for t in r]
        assert scores == sorted(scores, reverse=True)
        assert all(0 < s <= 1 for s in scores)


def test_ranker_prefers_full_waves():
    """With 256 CUs and one workgroup per CU, a problem of exactly 256
    256x256 tiles fills one wave; the same problem in 128x128 tiles (1024
    tiles, two per CU) also fills whole waves, so only tile efficiency
    separates them and the large tile wins.  At 257 tiles the large tile
    pays a second, nearly empty wave."""
    full = fgg.rank_tiles(fgg.FP8, 256 * 16, 256 * 16, 1024, 1, num_cus=256)
    assert (full[0]["block_m"], full[0]["block_n"]) == (256, 256)
    ragged = fgg.rank_tiles(fgg.FP8, 256 * 16 + 1, 256 * 16, 1024, 1, num_cus=256)
    top = ragged[0]
    assert (top["block_m"], top["block_n"]) != (256, 256)


def test_ranker_run_align():
    """c3's shape (G=32 experts in M=16384 rows, N=2048): without a promise
    every expert boundary is charged to a window of any height, and 128x256
    and 256x256 score within a few percent of each other; with runs aligned
    to 128 rows the 128-row tiles carry no two-expert windows and 128x256
    ranks first by a wide margin.  Alignment to 256 favours no 128-row shape
    over 256x256 again.  A dense problem (G=1) is unaffected."""
    def score(r, bm, bn):
        return next(t["score"] for t in r if (t["block_m"], t["block_n"]) == (bm, bn))
    plain = fgg.rank_tiles(fgg.FP8, 16384, 2048, 7168, 32, num_cus=256)
    assert abs(score(plain, 128, 256) / score(plain, 256, 256) - 1) < 0.05
    a128 = fgg.rank_tiles(fgg.FP8, 16384, 2048, 7168, 32, num_cus=256, run_align=128)
    assert (a128[0]["block_m"], a128[0]["block_n"]) == (128, 256)
    assert score(a128, 128, 256) > 1.2 * score(a128, 256, 256)
    assert score(a128, 256, 256) == score(plain, 256, 256)
    a256 = fgg.rank_tiles(fgg.FP8, 16384, 2048, 7168, 32, num_cus=256, run_align=256)
    assert (a256[0]["block_m"], a256[0]["block_n"]) == (256, 256)
    assert a256[0]["score"] > score(plain, 256, 256)
    dense = fgg.rank_tiles(fgg.FP4, 2048, 36864, 4608, 1, num_cus=256)
    assert dense == fgg.rank_tiles(fgg.FP4, 2048, 36864, 4608, 1, num_cus=256, run_align=128)
    lib = fgg.load_library()
    arr = (fgg._Tile * 4)()
    assert lib.fgg_rank_tiles_aligned(fgg.FP8, 64, 128, 128, 2, -1, 256, arr, 4) == -1
    assert "run_align" in lib.fgg_last_error().decode()


def test_device_info_without_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(ValueError):
        fgg.device_info()


def test_expand_quantizer_validation():
    lib = fgg.load_library()
    st = lib.quantize_fp8_1x128_rows(P, 0, P, P, 8, 4, 256, None)
    assert st == 1 and "rows" in lib.fgg_last_error().decode()
    assert lib.quantize_fp8_1x128_rows(P, P + 2, P, P, 8, 4, 256, None) == 3
    st = lib.quantize_fp8_1x128_rows(P, P, P, P, 8, 0, 256, None)
    assert st == 1 and "T" in lib.fgg_last_error().decode()
    assert lib.quantize_fp8_1x128_rows(P, P, P, P, 8, 4, 200, None) == 1
    st = lib.quantize_fp8_1x128_rows(P, P, P, P, 1 << 24, 4, 1 << 20, None)
    assert st == 2 and "2^31" in lib.fgg_last_error().decode()
    st = lib.quantize_nvfp4_static_rows(P, P, P, P, 0.0, 8, 4, 256, None)
    assert st == 1 and "global_scale" in lib.fgg_last_error().decode()
    assert lib.quantize_nvfp4_static_rows(P, P, P, P, 1.0, 8, 4, 144, None) == 2
    assert lib.quantize_nvfp4_static_rows(P + 8, P, P, P, 1.0, 8, 4, 256, None) == 3


def test_ranker_score_forms():
    """The kept score equals throughput / (rounds * slots * BM * BN) up to
    the constant M * N (a predicted-time form), where a last round with a
    fraction f of the slots busy counts 0.65 + 0.35 f; the literal page form
    also divides by tile_n and keeps num_waves whole.  Both rank every config;
    on a problem where every shape fills whole waves they can disagree only
    through tile_n."""
    for kind in (fgg.FP8, fgg.FP4):
        for (M, N, G) in ((8192, 4096, 8), (16384, 2048, 32), (2048, 36864, 1), (777, 256, 8)):
            kept = fgg.rank_tiles(kind, M, N, 7168, G, num_cus=256)
            for t in kept:
                bm, bn = t["block_m"], t["block_n"]
                windows = -(-M // bm)
                row_tiles = windows + min(G - 1, windows * 4)
                tiles = row_tiles * -(-N // bn)
                slots = 256 * t["wg_per_cu"]
                full, rem = divmod(tiles, slots)
                rounds = full + (0.65 + 0.35 * rem / slots if rem else 0.0)
                assert M <= row_tiles * bm  # m_eff <= 1: the identity below holds
                pred = M * N * t["tput"] / (bm * bn * rounds * slots)
                assert abs(t["score"] - pred) <= 1e-5 * max(1.0, pred)
            lit = fgg.rank_tiles(kind, M, N, 7168, G, num_cus=256, variant=fgg.SCORE_LITERAL)
            assert sorted(t["id"] for t in lit) == sorted(t["id"] for t in kept)
    lib = fgg.load_library()
    arr = (fgg._Tile * 4)()
    assert lib.fgg_rank_tiles_variant(fgg.FP8, 64, 128, 128, 2, 0, 7, 256, arr, 4) == -1
