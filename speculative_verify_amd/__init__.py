"""speculative_verify_amd -- low-bit linear layers for MI355X (gfx950).

A thin ctypes binding over ``libsvq.so`` (C ABI in ``include/svq.h``).  It
only marshals arguments: every step of the computation runs in the library's
HIP kernels (device calls) or its C++ packers (host calls).  PyTorch supplies
device memory and the current stream.  If the library is missing, every call
raises -- there is no fallback path.

Functions (same names as the C ABI):
  pack_int4_grouped, unpack_int4_grouped, pack_binary_planes,
  unpack_binary_planes, pack_sa, unpack_sa,
  quantize_int4_frozen, fit_binary_planes,
  snap_sa_scales                             host numpy arrays
  gemv_w4a16, gemv_binplane, gemv_sa, gemm_smallm_w4a16,
  gemm_smallm_binplane, gemm_smallm_sa,
  lmhead_argmax, lmhead_argmax_noalloc, lmhead_argmax_binplane,
  lmhead_verify_greedy, verify_greedy,
  svq_stream_read                            torch CUDA tensors
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "SvqError", "lib_path", "load", "int4_packed_bytes", "binplane_packed_bytes",
    "sa_packed_bytes", "lmhead_workspace_bytes", "pack_int4_grouped", "unpack_int4_grouped",
    "pack_binary_planes", "unpack_binary_planes", "pack_sa", "unpack_sa", "quantize_int4_frozen",
    "fit_binary_planes", "snap_sa_scales", "gemv_w4a16",
    "gemv_binplane", "gemv_sa", "gemm_smallm_w4a16", "gemm_smallm_binplane", "gemm_smallm_sa", "lmhead_argmax", "lmhead_argmax_binplane",
    "lmhead_verify_greedy", "lmhead_argmax_noalloc",
    "verify_greedy", "svq_stream_read",
]

GROUP = 128
ERRORS = {-1: "NULL", -2: "SHAPE", -3: "ALIGN", -4: "RANGE", -5: "WORKSPACE", -6: "HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class SvqError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: SVQ_ERR_{ERRORS.get(code, code)} ({code}): {msg}")
        self.code = code


def lib_path() -> str:
    return os.environ.get("SVQ_LIB", os.path.join(_HERE, "libsvq.so"))


def load():
    """Load libsvq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "or python speculative_verify_amd/build.py")
    lib = ctypes.CDLL(path)
    V, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "svq_last_error": ([], ctypes.c_char_p),
        "svq_int4_packed_bytes": ([I64, I64, I32], SZ),
        "svq_binplane_packed_bytes": ([I64, I64, I32, I32], SZ),
        "svq_sa_packed_bytes": ([I64, I64, I32, I32], SZ),
        "svq_lmhead_workspace_bytes": ([I32], SZ),
        "pack_int4_grouped": ([V, V, I64, I64, I32, V], ctypes.c_int),
        "unpack_int4_grouped": ([V, I64, I64, I32, V, V], ctypes.c_int),
        "pack_binary_planes": ([V, V, I64, I64, I32, I32, V], ctypes.c_int),
        "unpack_binary_planes": ([V, I64, I64, I32, I32, V, V], ctypes.c_int),
        "pack_sa": ([V, V, V, I64, I64, I32, I32, V], ctypes.c_int),
        "unpack_sa": ([V, I64, I64, I32, I32, V, V, V], ctypes.c_int),
        "quantize_int4_frozen": ([V, V, I64, I64, I32, V], ctypes.c_int),
        "fit_binary_planes": ([V, I64, I64, I32, I32, I32, V, V], ctypes.c_int),
        "snap_sa_scales": ([V, I64, I64, I32, I32, V, V], ctypes.c_int),
        "gemv_w4a16": ([V, V, V, I64, I64, I32, V], ctypes.c_int),
        "gemv_sa": ([V, V, V, I64, I64, I32, I32, V], ctypes.c_int),
        "gemm_smallm_sa": ([V, V, V, I32, I64, I64, I32, I32, V], ctypes.c_int),
        "gemv_binplane": ([V, V, V, I64, I64, I32, I32, V], ctypes.c_int),
        "gemm_smallm_w4a16": ([V, V, V, I32, I64, I64, I32, V], ctypes.c_int),
        "gemm_smallm_binplane": ([V, V, V, I32, I64, I64, I32, I32, V], ctypes.c_int),
        "lmhead_argmax": ([V, V, I32, I64, I64, I32, V, V, V, V, SZ, V], ctypes.c_int),
        "lmhead_argmax_noalloc": ([V, V, I32, I64, I64, I32, V, V, V, V], ctypes.c_int),
        "lmhead_verify_greedy": ([V, V, I32, I64, I64, I32, V, V, V, V, V, V, SZ, V], ctypes.c_int),
        "lmhead_argmax_binplane": ([V, V, I32, I64, I64, I32, I32, V, V, V, V, SZ, V], ctypes.c_int),
        "verify_greedy": ([V, V, I32, V, V], ctypes.c_int),
        "svq_stream_read": ([V, SZ, V, I32, V], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        msg = load().svq_last_error().decode(errors="replace")
        raise SvqError(fn, rc, msg)


def _np_ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dev_ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device argument must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError("device argument must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---- sizes ------------------------------------------------------------------

def int4_packed_bytes(N: int, K: int, G: int = GROUP) -> int:
    return int(load().svq_int4_packed_bytes(N, K, G))


def binplane_packed_bytes(N: int, K: int, P: int, G: int = GROUP) -> int:
    return int(load().svq_binplane_packed_bytes(N, K, G, P))


def sa_packed_bytes(N: int, K: int, P: int, G: int = GROUP) -> int:
    return int(load().svq_sa_packed_bytes(N, K, G, P))


def lmhead_workspace_bytes(M: int) -> int:
    return int(load().svq_lmhead_workspace_bytes(M))


# ---- host packers -------------------------------------------------------------

def pack_int4_grouped(codes: np.ndarray, scales_bf16: np.ndarray, G: int = GROUP) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.int8)
    scales = np.ascontiguousarray(scales_bf16, np.uint16)
    N, K = codes.shape
    out = np.empty(int4_packed_bytes(N, K, G), np.uint8)
    _check("pack_int4_grouped", load().pack_int4_grouped(_np_ptr(codes), _np_ptr(scales), N, K, G, _np_ptr(out)))
    return out


def unpack_int4_grouped(packed: np.ndarray, N: int, K: int, G: int = GROUP):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.empty((N, K), np.int8)
    scales = np.empty((N, K // G), np.uint16)
    _check("unpack_int4_grouped",
           load().unpack_int4_grouped(_np_ptr(packed), N, K, G, _np_ptr(codes), _np_ptr(scales)))
    return codes, scales


def pack_binary_planes(signs: np.ndarray, alpha_f16: np.ndarray, G: int = GROUP) -> np.ndarray:
    signs = np.ascontiguousarray(signs, np.int8)
    alpha = np.ascontiguousarray(alpha_f16, np.uint16)
    P, N, K = signs.shape
    out = np.empty(binplane_packed_bytes(N, K, P, G), np.uint8)
    _check("pack_binary_planes",
           load().pack_binary_planes(_np_ptr(signs), _np_ptr(alpha), N, K, G, P, _np_ptr(out)))
    return out


def unpack_binary_planes(packed: np.ndarray, N: int, K: int, P: int, G: int = GROUP):
    packed = np.ascontiguousarray(packed, np.uint8)
    signs = np.empty((P, N, K), np.int8)
    alpha = np.empty((P, N, K // G), np.uint16)
    _check("unpack_binary_planes",
           load().unpack_binary_planes(_np_ptr(packed), N, K, G, P, _np_ptr(signs), _np_ptr(alpha)))
    return signs, alpha


def pack_sa(signs: np.ndarray, codes: np.ndarray, d_f16: np.ndarray, G: int = GROUP) -> np.ndarray:
    signs = np.ascontiguousarray(signs, np.int8)
    codes = np.ascontiguousarray(codes, np.uint8)
    d = np.ascontiguousarray(d_f16, np.uint16)
    P, N, K = signs.shape
    out = np.empty(max(sa_packed_bytes(N, K, P, G), 1), np.uint8)
    _check("pack_sa", load().pack_sa(_np_ptr(signs), _np_ptr(codes), _np_ptr(d), N, K, G, P, _np_ptr(out)))
    return out


def unpack_sa(packed: np.ndarray, N: int, K: int, P: int, G: int = GROUP):
    packed = np.ascontiguousarray(packed, np.uint8)
    signs = np.empty((P, N, K), np.int8)
    codes = np.empty((P, N, K // G), np.uint8)
    d = np.empty((N, K // 256), np.uint16)
    _check("unpack_sa", load().unpack_sa(_np_ptr(packed), N, K, G, P, _np_ptr(signs), _np_ptr(codes), _np_ptr(d)))
    return signs, codes, d


def quantize_int4_frozen(w_bf16: np.ndarray, scales_bf16: np.ndarray, G: int = GROUP) -> np.ndarray:
    w = np.ascontiguousarray(w_bf16, np.uint16)
    s = np.ascontiguousarray(scales_bf16, np.uint16)
    N, K = w.shape
    codes = np.empty((N, K), np.int8)
    _check("quantize_int4_frozen", load().quantize_int4_frozen(_np_ptr(w), _np_ptr(s), N, K, G, _np_ptr(codes)))
    return codes


def fit_binary_planes(w_bf16: np.ndarray, P: int, G: int = GROUP, iters: int = 10):
    w = np.ascontiguousarray(w_bf16, np.uint16)
    N, K = w.shape
    signs = np.empty((P, N, K), np.int8)
    alpha = np.empty((P, N, K // G), np.uint16)
    _check("fit_binary_planes",
           load().fit_binary_planes(_np_ptr(w), N, K, G, P, iters, _np_ptr(signs), _np_ptr(alpha)))
    return signs, alpha


def snap_sa_scales(alpha_f16: np.ndarray, G: int = GROUP):
    a = np.ascontiguousarray(alpha_f16, np.uint16)
    P, N, ng = a.shape
    K = ng * G
    codes = np.empty((P, N, ng), np.uint8)
    d = np.empty((N, K // 256), np.uint16)
    _check("snap_sa_scales", load().snap_sa_scales(_np_ptr(a), N, K, G, P, _np_ptr(codes), _np_ptr(d)))
    return codes, d


# ---- device calls (torch tensors; bf16/fp16 values as int16/uint16 bits or bf16) --
#
# Every wrapper checks, before anything reaches the library, that each tensor
# holds at least the bytes the call reads or writes (numel * element_size),
# so an undersized tensor or a 1-byte dtype where 2-byte values are expected
# raises ValueError instead of turning into out-of-bounds device accesses.
# Shape errors the library itself reports (a size function returning 0) are
# left to the library.

def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _args(fn: str, *specs):
    """Device pointers of the (tensor, bytes needed, name) specs, after
    checking every tensor's size (all sizes first, then the pointers)."""
    for t, need, what in specs:
        if t is not None and need > 0 and _nbytes(t) < need:
            raise ValueError(f"{fn}: {what} holds {_nbytes(t)} bytes, the call needs {need}")
    return [_dev_ptr(t) for t, _, _ in specs]


def _int4_bytes(N, K, G):
    return int4_packed_bytes(N, K, G) if N >= 1 and K >= 1 else 0


def _plane_bytes(N, K, P, G):
    return binplane_packed_bytes(N, K, P, G) if N >= 1 and K >= 1 and 1 <= P <= 6 else 0


def _sa_bytes(N, K, P, G):
    return sa_packed_bytes(N, K, P, G) if N >= 1 and K >= 1 and 2 <= P <= 6 else 0


def _rows(M, L):
    return 2 * M * L if M >= 1 and L >= 1 else 0


def gemv_w4a16(packed, x, y, N: int, K: int, G: int = GROUP, stream=None) -> None:
    fn = "gemv_w4a16"
    pw, xp, yp = _args(fn, (packed, _int4_bytes(N, K, G), "packed"), (x, _rows(1, K), "x"), (y, _rows(1, N), "y"))
    _check(fn, load().gemv_w4a16(pw, xp, yp, N, K, G, _stream(stream)))


def gemv_binplane(packed, x, y, N: int, K: int, P: int, G: int = GROUP, stream=None) -> None:
    fn = "gemv_binplane"
    pw, xp, yp = _args(fn, (packed, _plane_bytes(N, K, P, G), "packed"), (x, _rows(1, K), "x"),
                       (y, _rows(1, N), "y"))
    _check(fn, load().gemv_binplane(pw, xp, yp, N, K, G, P, _stream(stream)))


def gemm_smallm_w4a16(packed, X, Y, M: int, N: int, K: int, G: int = GROUP, stream=None) -> None:
    fn = "gemm_smallm_w4a16"
    pw, xp, yp = _args(fn, (packed, _int4_bytes(N, K, G), "packed"), (X, _rows(M, K), "X"), (Y, _rows(M, N), "Y"))
    _check(fn, load().gemm_smallm_w4a16(pw, xp, yp, M, N, K, G, _stream(stream)))


def gemm_smallm_binplane(packed, X, Y, M: int, N: int, K: int, P: int, G: int = GROUP, stream=None) -> None:
    fn = "gemm_smallm_binplane"
    pw, xp, yp = _args(fn, (packed, _plane_bytes(N, K, P, G), "packed"), (X, _rows(M, K), "X"),
                       (Y, _rows(M, N), "Y"))
    _check(fn, load().gemm_smallm_binplane(pw, xp, yp, M, N, K, G, P, _stream(stream)))


def gemv_sa(packed, x, y, N: int, K: int, P: int, G: int = GROUP, stream=None) -> None:
    fn = "gemv_sa"
    pw, xp, yp = _args(fn, (packed, _sa_bytes(N, K, P, G), "packed"), (x, _rows(1, K), "x"), (y, _rows(1, N), "y"))
    _check(fn, load().gemv_sa(pw, xp, yp, N, K, G, P, _stream(stream)))


def gemm_smallm_sa(packed, X, Y, M: int, N: int, K: int, P: int, G: int = GROUP, stream=None) -> None:
    fn = "gemm_smallm_sa"
    pw, xp, yp = _args(fn, (packed, _sa_bytes(N, K, P, G), "packed"), (X, _rows(M, K), "X"), (Y, _rows(M, N), "Y"))
    _check(fn, load().gemm_smallm_sa(pw, xp, yp, M, N, K, G, P, _stream(stream)))


def _head_specs(M, N, K, X, argmax, maxlogit, row_ids):
    m = M if M >= 1 else 0
    return ((X, _rows(M, K), "X"), (row_ids, 4 * N if N >= 1 else 0, "row_ids"), (argmax, 4 * m, "argmax"),
            (maxlogit, 4 * m, "maxlogit"))


def _ws_size(workspace):
    return 0 if workspace is None else _nbytes(workspace)


def lmhead_argmax(packed, X, M: int, N: int, K: int, argmax, maxlogit, workspace,
                  row_ids=None, G: int = GROUP, stream=None) -> None:
    fn = "lmhead_argmax"
    pw, xp, rp, ip, mp, wp = _args(fn, (packed, _int4_bytes(N, K, G), "packed"),
                                   *_head_specs(M, N, K, X, argmax, maxlogit, row_ids), (workspace, 0, "workspace"))
    _check(fn, load().lmhead_argmax(pw, xp, M, N, K, G, rp, ip, mp, wp, _ws_size(workspace), _stream(stream)))


def lmhead_argmax_noalloc(packed, X, M: int, N: int, K: int, argmax, maxlogit, row_ids=None, G: int = GROUP,
                          stream=None) -> None:
    fn = "lmhead_argmax_noalloc"
    pw, xp, rp, ip, mp = _args(fn, (packed, _int4_bytes(N, K, G), "packed"),
                               *_head_specs(M, N, K, X, argmax, maxlogit, row_ids))
    _check(fn, load().lmhead_argmax_noalloc(pw, xp, M, N, K, G, rp, ip, mp, _stream(stream)))


def lmhead_argmax_binplane(packed, X, M: int, N: int, K: int, P: int, argmax, maxlogit, workspace,
                           row_ids=None, G: int = GROUP, stream=None) -> None:
    fn = "lmhead_argmax_binplane"
    pw, xp, rp, ip, mp, wp = _args(fn, (packed, _plane_bytes(N, K, P, G), "packed"),
                                   *_head_specs(M, N, K, X, argmax, maxlogit, row_ids), (workspace, 0, "workspace"))
    _check(fn, load().lmhead_argmax_binplane(pw, xp, M, N, K, G, P, rp, ip, mp, wp, _ws_size(workspace),
                                             _stream(stream)))


def lmhead_verify_greedy(packed, X, M: int, N: int, K: int, draft_ids, argmax, maxlogit, accept_len,
                         workspace, row_ids=None, G: int = GROUP, stream=None) -> None:
    fn = "lmhead_verify_greedy"
    pw, xp, rp, ip, mp, dp, ap, wp = _args(
        fn, (packed, _int4_bytes(N, K, G), "packed"), *_head_specs(M, N, K, X, argmax, maxlogit, row_ids),
        (draft_ids, 4 * (M - 1) if M > 1 else 0, "draft_ids"), (accept_len, 4, "accept_len"),
        (workspace, 0, "workspace"))
    _check(fn, load().lmhead_verify_greedy(pw, xp, M, N, K, G, rp, dp, ip, mp, ap, wp, _ws_size(workspace),
                                           _stream(stream)))


def verify_greedy(target_ids, draft_ids, M: int, accept_len, stream=None) -> None:
    fn = "verify_greedy"
    tp, dp, ap = _args(fn, (target_ids, 4 * M if M >= 1 else 0, "target_ids"),
                       (draft_ids, 4 * (M - 1) if M > 1 else 0, "draft_ids"), (accept_len, 4, "accept_len"))
    _check(fn, load().verify_greedy(tp, dp, M, ap, _stream(stream)))


def svq_stream_read(src, nbytes: int, sink, wgs_per_cu: int = 0, stream=None) -> None:
    fn = "svq_stream_read"
    cus = 0
    if sink is not None and getattr(sink, "is_cuda", False):
        import torch
        cus = torch.cuda.get_device_properties(sink.device).multi_processor_count
    sp, kp = _args(fn, (src, nbytes if nbytes > 0 else 0, "src"), (sink, 8 * cus * 4, "sink"))
    _check(fn, load().svq_stream_read(sp, nbytes, kp, wgs_per_cu, _stream(stream)))
