"""Block-scaled FP8 / NVFP4 (grouped) GEMM for AMD MI355X (gfx950).

Thin Python binding of ``libfgg.so`` (C ABI in include/fgg.h).  The functions
take PyTorch tensors only as device memory and streams: they check dtypes,
shapes and devices, derive the sizes, and pass raw pointers plus the current
HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.  If the library is not
built, every call raises ``ImportError`` (build it with
``python -m fp4_grouped_gemm_amd.build``).

Errors reported by the library (bad sizes, alignment, device) raise
``ValueError`` with the library's message.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "grouped_fp8_gemm", "fp4_gemm", "grouped_fp4_gemm", "quantize_fp8_1x128",
    "quantize_nvfp4", "grouped_fp8_gemm_tune", "fp4_gemm_tune", "grouped_fp4_gemm_tune",
    "tuned_tile", "tune_clear", "fp4_gemm_problems", "fp8_gemm_problems", "grouped_w4a16_gemm",
    "rank_tiles",
    "num_tiles",
    "device_info", "library_path", "load_library", "FP8", "FP4",
]

FP8, FP4 = 0, 1
# fgg_status values (include/fgg.h)
OK, EINVAL, EUNSUPPORTED, EALIGN, EDEVICE, EHIP = 0, 1, 2, 3, 4, 5
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libfgg.so")


class _Tile(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("waves", ctypes.c_int), ("wg_per_cu", ctypes.c_int), ("score", ctypes.c_float),
                ("tput", ctypes.c_float)]


SCORE_KEPT, SCORE_LITERAL = 0, 1  # FGG_SCORE_* (score forms of the ranker)


TUNE_MAX = 8  # FGG_TUNE_MAX


class _TuneReport(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("tile_id", ctypes.c_int * TUNE_MAX),
                ("ms", ctypes.c_float * TUNE_MAX), ("best", ctypes.c_int)]


MAX_PROBLEMS = 32  # FGG_MAX_PROBLEMS


class _Fp4Problem(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("a_scale", ctypes.c_void_p),
                ("b_scale", ctypes.c_void_p), ("C", ctypes.c_void_p), ("M", ctypes.c_int),
                ("N", ctypes.c_int), ("K", ctypes.c_int), ("alpha", ctypes.c_float)]


class _Fp8Problem(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("a_scale", ctypes.c_void_p),
                ("b_scale", ctypes.c_void_p), ("C", ctypes.c_void_p), ("M", ctypes.c_int),
                ("N", ctypes.c_int), ("K", ctypes.c_int)]


class _Options(ctypes.Structure):
    _fields_ = [("tile_id", ctypes.c_int), ("max_workgroups", ctypes.c_int),
                ("run_split", ctypes.c_int), ("run_align", ctypes.c_int)]


def load_library():
    """Load libfgg.so once and declare its C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp4_grouped_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    OPT = ctypes.POINTER(_Options)
    REP = ctypes.POINTER(_TuneReport)
    lib.fgg_last_error.restype = ctypes.c_char_p
    lib.fgg_last_error.argtypes = []
    for name, args in (
        ("grouped_fp8_gemm", [P, P, P, P, P, P, I, I, I, I, P]),
        ("grouped_fp8_gemm_ex", [P, P, P, P, P, P, I, I, I, I, OPT, P]),
        ("fp4_gemm", [P, P, P, P, F, P, I, I, I, P]),
        ("fp4_gemm_ex", [P, P, P, P, F, P, I, I, I, OPT, P]),
        ("grouped_fp4_gemm", [P, P, P, P, P, F, P, I, I, I, I, P]),
        ("grouped_fp4_gemm_ex", [P, P, P, P, P, F, P, I, I, I, I, OPT, P]),
        ("quantize_fp8_1x128", [P, P, P, I, I, P]),
        ("quantize_nvfp4", [P, P, P, P, I, I, P]),
        ("quantize_nvfp4_static", [P, P, P, F, I, I, P]),
        ("quantize_fp8_1x128_rows", [P, P, P, P, I, I, I, P]),
        ("quantize_nvfp4_static_rows", [P, P, P, P, F, I, I, I, P]),
        ("grouped_fp4_gemm_alpha", [P, P, P, P, P, P, P, I, I, I, I, P]),
        ("grouped_fp4_gemm_alpha_ex", [P, P, P, P, P, P, P, I, I, I, I, OPT, P]),
        ("fp4_gemm_problems", [ctypes.POINTER(_Fp4Problem), I, P]),
        ("fp8_gemm_problems", [ctypes.POINTER(_Fp8Problem), I, P]),
        ("fp8_gemm_problems_ex", [ctypes.POINTER(_Fp8Problem), I, OPT, P]),
        ("fp4_gemm_problems_ex", [ctypes.POINTER(_Fp4Problem), I, OPT, P]),
        ("grouped_w4a16_gemm", [P, P, P, P, F, P, I, I, I, I, P]),
        ("grouped_fp8_gemm_tune", [P, P, P, P, P, P, I, I, I, I, I, I, REP, OPT, P]),
        ("fp4_gemm_tune", [P, P, P, P, F, P, I, I, I, I, I, REP, OPT, P]),
        ("grouped_fp4_gemm_tune", [P, P, P, P, P, F, P, I, I, I, I, I, I, REP, OPT, P]),
        ("fgg_tuned_tile", [I, I, I, I, I]),
    ):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    lib.fgg_tune_clear.restype = None
    lib.fgg_tune_clear.argtypes = []
    lib.fgg_num_tiles.restype = I
    lib.fgg_num_tiles.argtypes = [I]
    lib.fgg_rank_tiles.restype = I
    lib.fgg_rank_tiles.argtypes = [I, I, I, I, I, I, ctypes.POINTER(_Tile), I]
    lib.fgg_rank_tiles_aligned.restype = I
    lib.fgg_rank_tiles_aligned.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(_Tile), I]
    lib.fgg_rank_tiles_variant.restype = I
    lib.fgg_rank_tiles_variant.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(_Tile), I]
    lib.fgg_device_info.restype = I
    lib.fgg_device_info.argtypes = [ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(I),
                                    ctypes.c_char_p, I]
    _LIB = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().fgg_last_error().decode(errors="replace")
        raise ValueError(msg or f"fgg status {status}")


def _opts(tile_id, max_workgroups, run_split=0, run_align=0):
    if tile_id is None and not max_workgroups and not run_split and not run_align:
        return None
    return ctypes.byref(_Options(-1 if tile_id is None else int(tile_id), int(max_workgroups or 0),
                                 int(run_split or 0), int(run_align or 0)))


def _torch():
    import torch  # imported lazily: the C-ABI checks need no torch
    return torch


def _bytes(t, name):
    """A device tensor of 8-bit codes viewed as uint8 (E4M3 / packed E2M1)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype not in (torch.uint8, torch.int8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        raise ValueError(f"{name} must hold 8-bit codes (uint8 / float8_e4m3fn), got {t.dtype}")
    return t.view(torch.uint8)


def _dev(t, name, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_ptr(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _out(out, M, N, device):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    if out.shape != (M, N) or out.dtype != torch.bfloat16:
        raise ValueError(f"out must be a bfloat16 tensor of shape ({M}, {N})")
    return _dev(out, "out", device)


def _fp8_call(A, B, a_scale, b_scale, m_indices, out):
    """Checks and marshals the arguments of grouped_fp8_gemm (and _tune)."""
    torch = _torch()
    A, B = _bytes(A, "A"), _bytes(B, "B")
    dev = A.device
    if A.dim() != 2 or B.dim() != 3:
        raise ValueError("A must be [M, K] and B [G, N, K]")
    M, K = A.shape
    G, N, Kb = B.shape
    if Kb != K:
        raise ValueError(f"A has K={K} but B has K={Kb}")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise ValueError("a_scale and b_scale must be float32")
    if tuple(a_scale.shape) != (M, K // 128) or tuple(b_scale.shape) != (G, N // 128, K // 128):
        raise ValueError(f"scale shapes must be ({M}, {K // 128}) and ({G}, {N // 128}, {K // 128})")
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError(f"m_indices must be int32 of shape ({M},)")
    for t, n in ((A, "A"), (B, "B"), (a_scale, "a_scale"), (b_scale, "b_scale"),
                 (m_indices, "m_indices")):
        _dev(t, n, dev)
    C = _out(out, M, N, dev)
    args = (A.data_ptr(), B.data_ptr(), a_scale.data_ptr(), b_scale.data_ptr(),
            m_indices.data_ptr(), C.data_ptr(), M, N, K, G)
    return C, dev, args


def grouped_fp8_gemm(A, B, a_scale, b_scale, m_indices, out=None, *, tile_id=None,
                     max_workgroups=0, run_split=0, run_align=0, stream=None):
    """C[M, N] (bfloat16) of the grouped block-scaled FP8 GEMM.

    A [M, K] and B [G, N, K] hold E4M3FN codes; a_scale [M, K/128] and
    b_scale [G, N/128, K/128] are float32; m_indices [M] is int32 (expert id or
    -1).  See include/fgg.h for the exact definition.  tile_id,
    max_workgroups, run_split and run_align are the fields of fgg_options
    (run_split: 0 automatic, -1 never, 1 always run each expert pass of a row
    window as its own workgroup; run_align > 0: every expert run starts at a
    multiple of that many rows, a hint for the tile choice).
    """
    torch = _torch()
    C, dev, args = _fp8_call(A, B, a_scale, b_scale, m_indices, out)
    with torch.cuda.device(dev):
        _check(load_library().grouped_fp8_gemm_ex(
            *args, _opts(tile_id, max_workgroups, run_split, run_align), _stream_ptr(stream, dev)))
    return C


def _report(r):
    return dict(tile_id=list(r.tile_id[:r.n]), ms=list(r.ms[:r.n]), best=r.best,
                chosen=r.tile_id[r.best] if r.n else -1)


def grouped_fp8_gemm_tune(A, B, a_scale, b_scale, m_indices, out=None, *, top_k=4, reps=5,
                          max_workgroups=0, run_split=0, run_align=0, stream=None):
    """Time the ranker's top_k tile configs on these inputs and record the
    fastest for this shape (C ABI grouped_fp8_gemm_tune; synchronises).
    run_align shapes the ranking the candidates come from; max_workgroups
    and run_split apply to every timed launch (as for grouped_fp8_gemm).
    Returns (C, report) with report = {tile_id, ms, best, chosen}."""
    torch = _torch()
    C, dev, args = _fp8_call(A, B, a_scale, b_scale, m_indices, out)
    rep = _TuneReport()
    with torch.cuda.device(dev):
        _check(load_library().grouped_fp8_gemm_tune(
            *args, int(top_k), int(reps), ctypes.byref(rep),
            _opts(None, max_workgroups, run_split, run_align), _stream_ptr(stream, dev)))
    return C, _report(rep)


def _fp4_shapes(A, a_scale, b_scale):
    torch = _torch()
    if a_scale.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        raise ValueError("NVFP4 scales must be E4M3 bytes (uint8 / float8_e4m3fn)")
    if b_scale.dtype != a_scale.dtype:
        raise ValueError("a_scale and b_scale must have the same dtype")
    M, K2 = A.shape
    return M, 2 * K2


def _fp4_call(A, B, a_scale, b_scale, m_indices, alpha, out):
    """Checks and marshals the arguments of fp4_gemm (m_indices None) or
    grouped_fp4_gemm (and their _tune variants)."""
    torch = _torch()
    A, B = _bytes(A, "A"), _bytes(B, "B")
    dev = A.device
    grouped = m_indices is not None
    if A.dim() != 2 or B.dim() != (3 if grouped else 2):
        raise ValueError("A must be [M, K/2] and B " + ("[G, N, K/2]" if grouped else "[N, K/2]"))
    M, K = _fp4_shapes(A, a_scale, b_scale)
    G, N, K2 = B.shape if grouped else (1, *B.shape)
    if K2 * 2 != K:
        raise ValueError("A and B disagree on K")
    sa, sb = _bytes(a_scale, "a_scale"), _bytes(b_scale, "b_scale")
    want_sb = (G, N, K // 16) if grouped else (N, K // 16)
    if tuple(sa.shape) != (M, K // 16) or tuple(sb.shape) != want_sb:
        raise ValueError(f"scale shapes must be ({M}, {K // 16}) and {want_sb}")
    tensors = [(A, "A"), (B, "B"), (sa, "a_scale"), (sb, "b_scale")]
    if grouped:
        if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
            raise ValueError(f"m_indices must be int32 of shape ({M},)")
        tensors.append((m_indices, "m_indices"))
    for t, n in tensors:
        _dev(t, n, dev)
    C = _out(out, M, N, dev)
    if grouped:
        args = (A.data_ptr(), B.data_ptr(), sa.data_ptr(), sb.data_ptr(), m_indices.data_ptr(),
                float(alpha), C.data_ptr(), M, N, K, G)
    else:
        args = (A.data_ptr(), B.data_ptr(), sa.data_ptr(), sb.data_ptr(), float(alpha),
                C.data_ptr(), M, N, K)
    return C, dev, args


def fp4_gemm(A, B, a_scale, b_scale, alpha, out=None, *, tile_id=None, max_workgroups=0,
             stream=None):
    """C[M, N] (bfloat16) of the dense NVFP4 GEMM: A [M, K/2] and B [N, K/2]
    packed E2M1, a_scale [M, K/16] and b_scale [N, K/16] E4M3 bytes, alpha =
    product of the two global scales."""
    torch = _torch()
    C, dev, args = _fp4_call(A, B, a_scale, b_scale, None, alpha, out)
    with torch.cuda.device(dev):
        _check(load_library().fp4_gemm_ex(*args, _opts(tile_id, max_workgroups),
                                          _stream_ptr(stream, dev)))
    return C


def grouped_fp4_gemm(A, B, a_scale, b_scale, m_indices, alpha, out=None, *, tile_id=None,
                     max_workgroups=0, run_split=0, run_align=0, stream=None):
    """C[M, N] (bfloat16) of the grouped NVFP4 GEMM: B [G, N, K/2], b_scale
    [G, N, K/16]; m_indices int32 [M] routes rows (-1 = padding).  alpha is
    a float (one global scale for every expert) or a float32 device tensor
    [G] of per-expert factors (C ABI grouped_fp4_gemm_alpha)."""
    torch = _torch()
    per_expert = isinstance(alpha, torch.Tensor)
    C, dev, args = _fp4_call(A, B, a_scale, b_scale, m_indices, 1.0 if per_expert else alpha, out)
    lib = load_library()
    with torch.cuda.device(dev):
        if per_expert:
            G = B.shape[0]
            if alpha.dtype != torch.float32 or tuple(alpha.shape) != (G,):
                raise ValueError(f"per-expert alpha must be a float32 tensor of shape ({G},)")
            _dev(alpha, "alpha", dev)
            a = list(args)
            a[5] = alpha.data_ptr()
            _check(lib.grouped_fp4_gemm_alpha_ex(
                *a, _opts(tile_id, max_workgroups, run_split, run_align), _stream_ptr(stream, dev)))
        else:
            _check(lib.grouped_fp4_gemm_ex(
                *args, _opts(tile_id, max_workgroups, run_split, run_align),
                _stream_ptr(stream, dev)))
    return C


def grouped_w4a16_gemm(A, B, b_scale, m_indices, b_global, out=None, *, stream=None):
    """C[M, N] (bfloat16) of the grouped W4A16 GEMM (decode path): A [M, K]
    bfloat16 activations, B [G, N, K/2] packed E2M1, b_scale [G, N, K/16] E4M3
    bytes, m_indices int32 [M], b_global the FP32 global scale of B."""
    torch = _torch()
    if not isinstance(A, torch.Tensor) or A.dtype != torch.bfloat16 or A.dim() != 2:
        raise ValueError("A must be a 2-D torch.bfloat16 tensor [M, K]")
    dev = A.device
    B, sb = _bytes(B, "B"), _bytes(b_scale, "b_scale")
    M, K = A.shape
    if B.dim() != 3 or B.shape[2] * 2 != K:
        raise ValueError(f"B must be [G, N, {K // 2}]")
    G, N, _ = B.shape
    if tuple(sb.shape) != (G, N, K // 16):
        raise ValueError(f"b_scale must be ({G}, {N}, {K // 16})")
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError(f"m_indices must be int32 of shape ({M},)")
    for t, n in ((A, "A"), (B, "B"), (sb, "b_scale"), (m_indices, "m_indices")):
        _dev(t, n, dev)
    C = _out(out, M, N, dev)
    with torch.cuda.device(dev):
        _check(load_library().grouped_w4a16_gemm(A.data_ptr(), B.data_ptr(), sb.data_ptr(),
                                                 m_indices.data_ptr(), float(b_global),
                                                 C.data_ptr(), M, N, K, G,
                                                 _stream_ptr(stream, dev)))
    return C


def fp4_gemm_problems(problems, outs=None, *, tile_id=None, max_workgroups=0, stream=None):
    """A batch of dense NVFP4 GEMMs of different shapes in one launch (C ABI
    fp4_gemm_problems).  ``problems``: sequence of (A, B, a_scale, b_scale,
    alpha) as for fp4_gemm; returns the list of C tensors."""
    torch = _torch()
    if not 1 <= len(problems) <= MAX_PROBLEMS:
        raise ValueError(f"need 1 to {MAX_PROBLEMS} problems, got {len(problems)}")
    arr = (_Fp4Problem * len(problems))()
    Cs, dev = [], None
    for g, (A, B, a_scale, b_scale, alpha) in enumerate(problems):
        C, d, args = _fp4_call(A, B, a_scale, b_scale, None, alpha,
                               None if outs is None else outs[g])
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError("all problems must be on one device")
        a_ptr, b_ptr, sa_ptr, sb_ptr, al, c_ptr, M, N, K = args
        arr[g] = _Fp4Problem(a_ptr, b_ptr, sa_ptr, sb_ptr, c_ptr, M, N, K, al)
        Cs.append(C)
    with torch.cuda.device(dev):
        _check(load_library().fp4_gemm_problems_ex(arr, len(problems),
                                                   _opts(tile_id, max_workgroups),
                                                   _stream_ptr(stream, dev)))
    return Cs


def fp8_gemm_problems(problems, outs=None, *, tile_id=None, max_workgroups=0, stream=None):
    """A batch of dense block-scaled FP8 GEMMs of different shapes in one
    launch (C ABI fp8_gemm_problems).  ``problems``: sequence of (A [M, K],
    B [N, K], a_scale [M, K/128] float32, b_scale [N/128, K/128] float32),
    A and B holding E4M3FN codes; returns the list of C tensors (bfloat16)."""
    torch = _torch()
    if not 1 <= len(problems) <= MAX_PROBLEMS:
        raise ValueError(f"need 1 to {MAX_PROBLEMS} problems, got {len(problems)}")
    arr = (_Fp8Problem * len(problems))()
    Cs, dev = [], None
    for g, (A, B, a_scale, b_scale) in enumerate(problems):
        A, B = _bytes(A, "A"), _bytes(B, "B")
        if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
            raise ValueError(f"problem {g}: A must be [M, K] and B [N, K]")
        M, K = A.shape
        N = B.shape[0]
        if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
            raise ValueError(f"problem {g}: a_scale and b_scale must be float32")
        if tuple(a_scale.shape) != (M, K // 128) or tuple(b_scale.shape) != (N // 128, K // 128):
            raise ValueError(f"problem {g}: scale shapes must be ({M}, {K // 128}) and "
                             f"({N // 128}, {K // 128})")
        d = A.device
        for t, n in ((B, "B"), (a_scale, "a_scale"), (b_scale, "b_scale")):
            _dev(t, n, d)
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError("all problems must be on one device")
        C = _out(None if outs is None else outs[g], M, N, d)
        arr[g] = _Fp8Problem(A.data_ptr(), B.data_ptr(), a_scale.data_ptr(), b_scale.data_ptr(),
                             C.data_ptr(), M, N, K)
        Cs.append(C)
    with torch.cuda.device(dev):
        _check(load_library().fp8_gemm_problems_ex(arr, len(problems),
                                                   _opts(tile_id, max_workgroups),
                                                   _stream_ptr(stream, dev)))
    return Cs


def fp4_gemm_tune(A, B, a_scale, b_scale, alpha, out=None, *, top_k=4, reps=5,
                  max_workgroups=0, stream=None):
    """Bounded autotune of fp4_gemm for this shape (as grouped_fp8_gemm_tune)."""
    torch = _torch()
    C, dev, args = _fp4_call(A, B, a_scale, b_scale, None, alpha, out)
    rep = _TuneReport()
    with torch.cuda.device(dev):
        _check(load_library().fp4_gemm_tune(*args, int(top_k), int(reps), ctypes.byref(rep),
                                            _opts(None, max_workgroups),
                                            _stream_ptr(stream, dev)))
    return C, _report(rep)


def grouped_fp4_gemm_tune(A, B, a_scale, b_scale, m_indices, alpha, out=None, *, top_k=4, reps=5,
                          max_workgroups=0, run_split=0, run_align=0, stream=None):
    """Bounded autotune of grouped_fp4_gemm for this shape (as
    grouped_fp8_gemm_tune)."""
    torch = _torch()
    C, dev, args = _fp4_call(A, B, a_scale, b_scale, m_indices, alpha, out)
    rep = _TuneReport()
    with torch.cuda.device(dev):
        _check(load_library().grouped_fp4_gemm_tune(
            *args, int(top_k), int(reps), ctypes.byref(rep),
            _opts(None, max_workgroups, run_split, run_align), _stream_ptr(stream, dev)))
    return C, _report(rep)


def tuned_tile(kind: int, M: int, N: int, K: int, G: int = 1) -> int:
    """The tile config recorded by a *_tune call for this shape, or -1."""
    return load_library().fgg_tuned_tile(kind, M, N, K, G)


def tune_clear() -> None:
    """Forget every recorded tuning choice (C ABI fgg_tune_clear)."""
    load_library().fgg_tune_clear()


def num_tiles(kind: int) -> int:
    return load_library().fgg_num_tiles(kind)


def rank_tiles(kind: int, M: int, N: int, K: int, G: int = 1, num_cus: int = 256,
               run_align: int = 0, variant: int = SCORE_KEPT):
    """The ranker's ordered tile configs for a problem (host logic only);
    run_align as in fgg_options; variant selects the score form
    (SCORE_KEPT, the one the entry points use, or SCORE_LITERAL)."""
    lib = load_library()
    n = max(1, lib.fgg_num_tiles(kind))
    arr = (_Tile * n)()
    k = lib.fgg_rank_tiles_variant(kind, M, N, K, G, run_align, variant, num_cus, arr, n)
    if k < 0:
        _check(1)
    return [dict(id=t.id, block_m=t.block_m, block_n=t.block_n, waves=t.waves,
                 wg_per_cu=t.wg_per_cu, score=t.score, tput=t.tput) for t in arr[:k]]


def device_info():
    lib = load_library()
    cu, lds, clk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    arch = ctypes.create_string_buffer(64)
    _check(lib.fgg_device_info(ctypes.byref(cu), ctypes.byref(lds), ctypes.byref(clk), arch, 64))
    return dict(num_cus=cu.value, lds_per_block=lds.value, clock_khz=clk.value,
                arch=arch.value.decode())


def _bf16_matrix(X):
    torch = _torch()
    if not isinstance(X, torch.Tensor) or X.dtype != torch.bfloat16 or X.dim() != 2:
        raise ValueError("X must be a 2-D torch.bfloat16 tensor [M, K]")
    return _dev(X, "X", X.device)


def _row_map(rows, X):
    torch = _torch()
    if rows.dtype != torch.int32 or rows.dim() != 1:
        raise ValueError("rows must be a 1-D int32 tensor")
    return _dev(rows, "rows", X.device)


def quantize_fp8_1x128(X, stream=None, rows=None):
    """BF16 activations [M, K] -> (E4M3FN codes uint8 [M, K], FP32 scales
    [M, K/128]): the A operand of grouped_fp8_gemm (C ABI quantize_fp8_1x128).

    rows (int32 [R], optional): the MoE row expansion fused in -- output row
    r quantises X[rows[r]], a padding row (zeros) where rows[r] is outside
    [0, M); the result has R rows (C ABI quantize_fp8_1x128_rows)."""
    torch = _torch()
    lib = load_library()
    X = _bf16_matrix(X)
    M, K = X.shape
    R = M if rows is None else rows.shape[0]
    Q = torch.empty((R, K), dtype=torch.uint8, device=X.device)
    S = torch.empty((R, max(K // 128, 1)), dtype=torch.float32, device=X.device)
    with torch.cuda.device(X.device):
        if rows is None:
            _check(lib.quantize_fp8_1x128(X.data_ptr(), Q.data_ptr(), S.data_ptr(), M, K,
                                          _stream_ptr(stream, X.device)))
        else:
            rows = _row_map(rows, X)
            _check(lib.quantize_fp8_1x128_rows(X.data_ptr(), rows.data_ptr(), Q.data_ptr(),
                                               S.data_ptr(), R, M, K,
                                               _stream_ptr(stream, X.device)))
    return Q, S


def quantize_nvfp4(X, stream=None, global_scale=None, rows=None):
    """BF16 activations [M, K] -> (packed E2M1 uint8 [M, K/2], E4M3FN scale
    codes uint8 [M, K/16], FP32 global scale as a 1-element device tensor):
    the A operand of fp4_gemm / grouped_fp4_gemm, whose alpha is this global
    scale times B's (C ABI quantize_nvfp4; no host synchronisation).

    global_scale: None computes g = amax(X) / 2688 on the device; a Python
    float is a calibrated, static g (C ABI quantize_nvfp4_static: one pass
    over X, block amaxes above 448 * 6 * g saturate).

    rows (int32 [R], optional; needs a static global_scale): the MoE row
    expansion fused in, as for quantize_fp8_1x128 (C ABI
    quantize_nvfp4_static_rows)."""
    torch = _torch()
    lib = load_library()
    X = _bf16_matrix(X)
    M, K = X.shape
    R = M if rows is None else rows.shape[0]
    Q = torch.empty((R, K // 2), dtype=torch.uint8, device=X.device)
    S = torch.empty((R, max(K // 16, 1)), dtype=torch.uint8, device=X.device)
    with torch.cuda.device(X.device):
        if rows is not None:
            if global_scale is None:
                raise ValueError("the row-expansion variant needs a static global_scale")
            gs = float(global_scale)
            rows = _row_map(rows, X)
            _check(lib.quantize_nvfp4_static_rows(X.data_ptr(), rows.data_ptr(), Q.data_ptr(),
                                                  S.data_ptr(), gs, R, M, K,
                                                  _stream_ptr(stream, X.device)))
            g = torch.full((1,), gs, dtype=torch.float32, device=X.device)
        elif global_scale is None:
            g = torch.empty((1,), dtype=torch.float32, device=X.device)
            _check(lib.quantize_nvfp4(X.data_ptr(), Q.data_ptr(), S.data_ptr(), g.data_ptr(),
                                      M, K, _stream_ptr(stream, X.device)))
        else:
            gs = float(global_scale)
            _check(lib.quantize_nvfp4_static(X.data_ptr(), Q.data_ptr(), S.data_ptr(), gs, M, K,
                                             _stream_ptr(stream, X.device)))
            g = torch.full((1,), gs, dtype=torch.float32, device=X.device)
    return Q, S, g
