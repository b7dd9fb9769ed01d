"""CPU fp64 oracle for the low-bit linear layers -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It loads ``liboracle.so`` (plain C,
built from ``oracle.c`` with gcc) and shares no code with the HIP library in
``speculative_verify_amd``; neither side imports the other.

Every function takes the *unpacked* definition (codes/signs, scales, bf16
activations) and returns fp64 results:

* ``linear_w4a16``    y = sum_g s[n,g] sum_{k in g} c[n,k] x[k]
  (Efficient Qwen Competition report, sec. 2.1 and 3.3: INT4 codes times
  frozen symmetric per-group scales, group 128 along the input dimension);
* ``linear_binplane`` y = sum_g sum_p alpha[p,n,g] sum_{k in g} b[p,n,k] x[k]
  (ShiftAddQwen README, intro and "Format");
* ``linear_sa``       the same sum with alpha[p,n,g] = d[n, g*G/256] * a[p,n,g]:
  u8 scale codes per (plane, group) and one fp16 d per 256-weight
  super-block (ShiftAddQwen README, "Method / Format", the sa* types);
* ``requant_int4``, ``fit_planes``, ``snap_sa``: the offline steps --
  frozen-grid INT4 requantisation (report sec. 2.1), the greedy + ALS
  sign-plane fit (README "Output-aware fit") and the snap of plane scales
  onto the sa* u8 grid (README "Format", "Scale distillation");
* ``argmax_w4a16``    greedy token = lowest index attaining the max logit
  (DFlash summary sec. 4.1; MTP study sec. 3.3 for the trimmed-head row map);
* ``pack_int4`` / ``pack_binplane`` / ``pack_sa`` state the packed byte layouts element by
  element (the pages name the formats, the layout is this project's own).

Each returned ``a`` array is sum_k |w[n,k] x[k]|, the scale of the stated
tolerance |y_gpu - y| <= 2e-3 * a + 1e-5.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_f16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_value.restype = ctypes.c_double
    lib.oracle_bf16_values.argtypes = [P, I64, P]
    lib.oracle_f16_values.argtypes = [P, I64, P]
    lib.oracle_linear_w4a16.argtypes = [P, P, P, I64, I64, I64, I64, P, P]
    lib.oracle_linear_w4a16.restype = ctypes.c_int
    lib.oracle_linear_binplane.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, P]
    lib.oracle_linear_binplane.restype = ctypes.c_int
    lib.oracle_linear_sa.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P, P]
    lib.oracle_linear_sa.restype = ctypes.c_int
    lib.oracle_sa_blob_bytes.argtypes = [I64, I64, I64, I64]
    lib.oracle_sa_blob_bytes.restype = I64
    lib.oracle_pack_sa.argtypes = [P, P, P, I64, I64, I64, I64, P]
    lib.oracle_pack_sa.restype = ctypes.c_int
    lib.oracle_f16_bits.argtypes = [ctypes.c_double]
    lib.oracle_f16_bits.restype = ctypes.c_uint16
    lib.oracle_requant_int4.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_requant_int4.restype = ctypes.c_int
    lib.oracle_fit_planes.argtypes = [P, I64, I64, I64, I64, I64, P, P, P]
    lib.oracle_fit_planes.restype = ctypes.c_int
    lib.oracle_snap_sa.argtypes = [P, I64, I64, I64, I64, P, P]
    lib.oracle_snap_sa.restype = ctypes.c_int
    lib.oracle_argmax_w4a16.argtypes = [P, P, P, I64, I64, I64, I64, P, P, P, P, P, P]
    lib.oracle_argmax_w4a16.restype = ctypes.c_int
    lib.oracle_argmax_binplane.argtypes = [P, P, P, I64, I64, I64, I64, I64, P, P, P, P, P, P]
    lib.oracle_argmax_binplane.restype = ctypes.c_int
    lib.oracle_verify_greedy.argtypes = [P, P, I64]
    lib.oracle_verify_greedy.restype = ctypes.c_int
    lib.oracle_int4_blob_bytes.argtypes = [I64, I64]
    lib.oracle_int4_blob_bytes.restype = I64
    lib.oracle_binplane_blob_bytes.argtypes = [I64, I64, I64]
    lib.oracle_binplane_blob_bytes.restype = I64
    lib.oracle_pack_int4.argtypes = [P, P, I64, I64, P]
    lib.oracle_pack_int4.restype = ctypes.c_int
    lib.oracle_pack_binplane.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_pack_binplane.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def bf16_values(bits) -> np.ndarray:
    """fp64 value of each bf16 bit pattern."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_bf16_values(_ptr(bits), bits.size, _ptr(out))
    return out


def f16_values(bits) -> np.ndarray:
    """fp64 value of each IEEE binary16 bit pattern."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_f16_values(_ptr(bits), bits.size, _ptr(out))
    return out


def linear_w4a16(codes, scales, x, G: int = 128):
    """(y, a) fp64 [M][N] for codes [N][K] int8, scales [N][K/G] bf16 bits,
    x [M][K] (or [K]) bf16 bits."""
    codes = _c(codes, np.int8)
    scales = _c(scales, np.uint16)
    x2 = _c(np.atleast_2d(x), np.uint16)
    N, K = codes.shape
    M = x2.shape[0]
    assert x2.shape[1] == K and scales.shape == (N, K // G)
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    rc = _load().oracle_linear_w4a16(_ptr(codes), _ptr(scales), _ptr(x2), M, N, K, G,
                                     _ptr(y), _ptr(a))
    if rc:
        raise ValueError(f"oracle_linear_w4a16 rc={rc}")
    return y, a


def linear_binplane(signs, alpha, x, G: int = 128):
    """(y, a) fp64 [M][N] for signs [P][N][K] in {-1,+1}, alpha [P][N][K/G]
    fp16 bits, x [M][K] bf16 bits."""
    signs = _c(signs, np.int8)
    alpha = _c(alpha, np.uint16)
    x2 = _c(np.atleast_2d(x), np.uint16)
    P, N, K = signs.shape
    M = x2.shape[0]
    assert x2.shape[1] == K and alpha.shape == (P, N, K // G)
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    rc = _load().oracle_linear_binplane(_ptr(signs), _ptr(alpha), _ptr(x2), M, N, K, G, P,
                                        _ptr(y), _ptr(a))
    if rc:
        raise ValueError(f"oracle_linear_binplane rc={rc}")
    return y, a


def linear_sa(signs, codes, d, x, G: int = 128):
    """(y, a) fp64 [M][N] for signs [P][N][K] in {-1,+1}, u8 scale codes
    [P][N][K/G], fp16 super-block scales d [N][K/256] (bits), x [M][K] bf16."""
    signs = _c(signs, np.int8)
    codes = _c(codes, np.uint8)
    d = _c(d, np.uint16)
    x2 = _c(np.atleast_2d(x), np.uint16)
    P, N, K = signs.shape
    M = x2.shape[0]
    assert x2.shape[1] == K and codes.shape == (P, N, K // G) and d.shape == (N, K // 256)
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    rc = _load().oracle_linear_sa(_ptr(signs), _ptr(codes), _ptr(d), _ptr(x2), M, N, K, G, P,
                                  _ptr(y), _ptr(a))
    if rc:
        raise ValueError(f"oracle_linear_sa rc={rc}")
    return y, a


def argmax_w4a16(codes, scales, x, G: int = 128, row_ids=None):
    """dict(out, idx, zmax, amax, zsecond), each of length M."""
    codes = _c(codes, np.int8)
    scales = _c(scales, np.uint16)
    x2 = _c(np.atleast_2d(x), np.uint16)
    N, K = codes.shape
    M = x2.shape[0]
    rid = None if row_ids is None else _c(row_ids, np.int32)
    out = np.empty(M, np.int32)
    idx = np.empty(M, np.int32)
    zmax = np.empty(M, np.float64)
    amax = np.empty(M, np.float64)
    zsec = np.empty(M, np.float64)
    rc = _load().oracle_argmax_w4a16(
        _ptr(codes), _ptr(scales), _ptr(x2), M, N, K, G,
        None if rid is None else _ptr(rid), _ptr(out), _ptr(idx), _ptr(zmax),
        _ptr(amax), _ptr(zsec))
    if rc:
        raise ValueError(f"oracle_argmax_w4a16 rc={rc}")
    return dict(out=out, idx=idx, zmax=zmax, amax=amax, zsecond=zsec)


def argmax_binplane(signs, alpha, x, G: int = 128, row_ids=None):
    """dict(out, idx, zmax, amax, zsecond) for a sign-plane head."""
    signs = _c(signs, np.int8)
    alpha = _c(alpha, np.uint16)
    x2 = _c(np.atleast_2d(x), np.uint16)
    P, N, K = signs.shape
    M = x2.shape[0]
    rid = None if row_ids is None else _c(row_ids, np.int32)
    out = np.empty(M, np.int32)
    idx = np.empty(M, np.int32)
    zmax = np.empty(M, np.float64)
    amax = np.empty(M, np.float64)
    zsec = np.empty(M, np.float64)
    rc = _load().oracle_argmax_binplane(
        _ptr(signs), _ptr(alpha), _ptr(x2), M, N, K, G, P,
        None if rid is None else _ptr(rid), _ptr(out), _ptr(idx), _ptr(zmax),
        _ptr(amax), _ptr(zsec))
    if rc:
        raise ValueError(f"oracle_argmax_binplane rc={rc}")
    return dict(out=out, idx=idx, zmax=zmax, amax=amax, zsecond=zsec)


def verify_greedy(target, draft) -> int:
    """tau for target tokens [M] and drafted tokens [M-1]."""
    t = _c(np.atleast_1d(target), np.int32)
    M = t.shape[0]
    d = _c(np.atleast_1d(draft) if M > 1 else np.zeros(1, np.int32), np.int32)
    if M > 1 and d.shape[0] != M - 1:
        raise ValueError("draft must hold M - 1 tokens")
    return int(_load().oracle_verify_greedy(_ptr(t), _ptr(d), M))


def pack_int4(codes, scales) -> np.ndarray:
    """Packed INT4 blob (uint8) per the element-wise layout statement."""
    codes = _c(codes, np.int8)
    scales = _c(scales, np.uint16)
    N, K = codes.shape
    lib = _load()
    blob = np.empty(int(lib.oracle_int4_blob_bytes(N, K)), np.uint8)
    rc = lib.oracle_pack_int4(_ptr(codes), _ptr(scales), N, K, _ptr(blob))
    if rc:
        raise ValueError(f"oracle_pack_int4 rc={rc}")
    return blob


def pack_binplane(signs, alpha) -> np.ndarray:
    """Packed binary-plane blob (uint8) per the element-wise layout statement."""
    signs = _c(signs, np.int8)
    alpha = _c(alpha, np.uint16)
    P, N, K = signs.shape
    lib = _load()
    blob = np.empty(int(lib.oracle_binplane_blob_bytes(N, K, P)), np.uint8)
    rc = lib.oracle_pack_binplane(_ptr(signs), _ptr(alpha), N, K, P, _ptr(blob))
    if rc:
        raise ValueError(f"oracle_pack_binplane rc={rc}")
    return blob


def pack_sa(signs, codes, d, G: int = 128) -> np.ndarray:
    """Packed sa blob (uint8) per the element-wise layout statement."""
    signs = _c(signs, np.int8)
    codes = _c(codes, np.uint8)
    d = _c(d, np.uint16)
    P, N, K = signs.shape
    lib = _load()
    blob = np.empty(int(lib.oracle_sa_blob_bytes(N, K, G, P)), np.uint8)
    rc = lib.oracle_pack_sa(_ptr(signs), _ptr(codes), _ptr(d), N, K, G, P, _ptr(blob))
    if rc:
        raise ValueError(f"oracle_pack_sa rc={rc}")
    return blob


def f16_bits(values) -> np.ndarray:
    """IEEE binary16 bits of fp64 values, round to nearest even."""
    lib = _load()
    v = np.atleast_1d(np.asarray(values, np.float64))
    return np.array([lib.oracle_f16_bits(float(x)) for x in v.ravel()], np.uint16).reshape(v.shape)


def requant_int4(w, scales, G: int = 128) -> np.ndarray:
    """INT4 codes [N][K] of bf16 weights w under frozen bf16 scales [N][K/G]."""
    w = _c(w, np.uint16)
    scales = _c(scales, np.uint16)
    N, K = w.shape
    assert scales.shape == (N, K // G)
    codes = np.empty((N, K), np.int8)
    rc = _load().oracle_requant_int4(_ptr(w), _ptr(scales), N, K, G, _ptr(codes))
    if rc:
        raise ValueError(f"oracle_requant_int4 rc={rc}")
    return codes


def fit_planes(w, P: int, G: int = 128, iters: int = 10):
    """(signs [P][N][K], alpha fp64 [P][N][K/G], alpha fp16 bits) fitted to
    bf16 weights w [N][K]: greedy init, then `iters` ALS rounds."""
    w = _c(w, np.uint16)
    N, K = w.shape
    signs = np.empty((P, N, K), np.int8)
    a64 = np.empty((P, N, K // G), np.float64)
    a16 = np.empty((P, N, K // G), np.uint16)
    rc = _load().oracle_fit_planes(_ptr(w), N, K, G, P, iters, _ptr(signs), _ptr(a64), _ptr(a16))
    if rc:
        raise ValueError(f"oracle_fit_planes rc={rc}")
    return signs, a64, a16


def snap_sa(alpha16, G: int = 128):
    """(codes u8 [P][N][K/G], d fp16 bits [N][K/256]) for fp16 plane scales."""
    alpha16 = _c(alpha16, np.uint16)
    P, N, ng = alpha16.shape
    K = ng * G
    codes = np.empty((P, N, ng), np.uint8)
    d = np.empty((N, K // 256), np.uint16)
    rc = _load().oracle_snap_sa(_ptr(alpha16), N, K, G, P, _ptr(codes), _ptr(d))
    if rc:
        raise ValueError(f"oracle_snap_sa rc={rc}")
    return codes, d
