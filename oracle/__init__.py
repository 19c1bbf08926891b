"""CPU oracle for the fused SwiGLU MLP (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The GPU library never calls it, and it calls nothing of the
GPU library: the two share no code.

`oracle.c` holds the arithmetic (fp64, plain loops); this module only loads
it with ctypes and marshals NumPy arrays.  `brute.py` is a second, pure-Python
implementation for tiny shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
F64 = 2

_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc build of an oracle source: IEEE fp64, no FMA contraction, OpenMP
    over independent output elements."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (when missing or stale)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def _bind(lib):
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_swiglu_rows.restype = ctypes.c_int
    lib.oracle_swiglu_rows.argtypes = [ctypes.c_int, vp, vp, vp, i64, i64, i64,
                                       vp, i64, dp, dp, dp, ctypes.c_int]
    lib.oracle_mlp_rows.restype = ctypes.c_int
    lib.oracle_mlp_rows.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64,
                                    vp, i64, dp, dp, ctypes.c_int]
    lib.oracle_default_threads.restype = ctypes.c_int
    lib.oracle_default_threads.argtypes = []
    lib.oracle_bf16_array_to_double.restype = ctypes.c_int
    lib.oracle_bf16_array_to_double.argtypes = [vp, i64, dp]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_from_float.restype = ctypes.c_uint8
    lib.oracle_e4m3_from_float.argtypes = [ctypes.c_float]
    lib.oracle_quantize_e4m3_columns.restype = ctypes.c_int
    lib.oracle_quantize_e4m3_columns.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_e2m1_to_double.restype = ctypes.c_double
    lib.oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_from_double.restype = ctypes.c_uint8
    lib.oracle_e2m1_from_double.argtypes = [ctypes.c_double]
    lib.oracle_mx_shared_exponent.restype = ctypes.c_int
    lib.oracle_mx_shared_exponent.argtypes = [ctypes.c_double]
    lib.oracle_quantize_mxfp4_columns.restype = ctypes.c_int
    lib.oracle_quantize_mxfp4_columns.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_dequantize_mxfp4_columns.restype = ctypes.c_int
    lib.oracle_dequantize_mxfp4_columns.argtypes = [vp, vp, i64, i64, dp]
    lib.oracle_rmsnorm_rows.restype = ctypes.c_int
    lib.oracle_rmsnorm_rows.argtypes = [ctypes.c_int, vp, vp, ctypes.c_double, i64, i64, dp]
    lib.oracle_dequantize_e4m3_columns.restype = ctypes.c_int
    lib.oracle_dequantize_e4m3_columns.argtypes = [vp, vp, i64, i64, dp]
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError("oracle inputs are float32 or float64 arrays, or uint16 bf16 bit patterns")


def _check(x, wg, wu, wd=None):
    dt = _dtype_of(x)
    for w in (wg, wu) + ((wd,) if wd is not None else ()):
        if _dtype_of(w) != dt:
            raise TypeError("x and the weights must share one dtype")
    M, d = x.shape
    d2, dff = wg.shape
    if d2 != d or wu.shape != (d, dff) or (wd is not None and wd.shape != (dff, d)):
        raise ValueError("shape mismatch")
    return dt, M, d, dff


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, len(r)


def bf16_to_double(bits: int, lib=None) -> float:
    return (lib or _load()).oracle_bf16_to_double(bits)


def sigmoid(z: float, lib=None) -> float:
    return (lib or _load()).oracle_sigmoid(float(z))


def silu(z: float, lib=None) -> float:
    return (lib or _load()).oracle_silu(float(z))


def swiglu(x, wg, wu, rows=None, want_gu=False, nthreads=0, lib=None):
    """h = silu(x.Wg) * (x.Wu) in fp64 for the given rows of x (all rows if
    None).  With want_gu, also returns g and u."""
    x, wg, wu = (np.ascontiguousarray(a) for a in (x, wg, wu))
    dt, M, d, dff = _check(x, wg, wu)
    r, nrows = _rows_arg(rows, M)
    h = np.empty((nrows, dff), dtype=np.float64)
    g = np.empty_like(h) if want_gu else None
    u = np.empty_like(h) if want_gu else None
    rc = (lib or _load()).oracle_swiglu_rows(dt, _ptr(x), _ptr(wg), _ptr(wu), M, d, dff,
                                    _ptr(r), nrows, _ptr(g), _ptr(u), _ptr(h), nthreads)
    if rc != 0:
        raise ValueError("oracle_swiglu_rows failed (%d)" % rc)
    return (h, g, u) if want_gu else h


def mlp(x, wg, wu, wd, rows=None, want_h=False, nthreads=0, lib=None):
    """y = (silu(x.Wg) * (x.Wu)) . Wd in fp64 for the given rows of x."""
    x, wg, wu, wd = (np.ascontiguousarray(a) for a in (x, wg, wu, wd))
    dt, M, d, dff = _check(x, wg, wu, wd)
    r, nrows = _rows_arg(rows, M)
    y = np.empty((nrows, d), dtype=np.float64)
    h = np.empty((nrows, dff), dtype=np.float64) if want_h else None
    rc = (lib or _load()).oracle_mlp_rows(dt, _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), M, d, dff,
                                 _ptr(r), nrows, _ptr(h), _ptr(y), nthreads)
    if rc != 0:
        raise ValueError("oracle_mlp_rows failed (%d)" % rc)
    return (y, h) if want_h else y


def bf16_array_to_double(a, lib=None) -> np.ndarray:
    """Exact widening of a uint16 array of bf16 patterns."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    if (lib or _load()).oracle_bf16_array_to_double(_ptr(a), a.size, _ptr(out)) != 0:
        raise ValueError("oracle_bf16_array_to_double failed")
    return out


def e4m3_to_double(code: int, lib=None) -> float:
    return (lib or _load()).oracle_e4m3_to_double(int(code))


def e4m3_from_float(v: float, lib=None) -> int:
    """Nearest E4M3 code (ties to even, saturating) of the fp32 value v."""
    return (lib or _load()).oracle_e4m3_from_float(float(np.float32(v)))


def quantize_e4m3(w, lib=None):
    """Per-column E4M3 quantisation of a K x N bf16 matrix (uint16 bits):
    returns (codes uint8 K x N, scales float32 N)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    K, N = w.shape
    codes = np.empty((K, N), dtype=np.uint8)
    scales = np.empty(N, dtype=np.float32)
    if (lib or _load()).oracle_quantize_e4m3_columns(_ptr(w), K, N, _ptr(codes), _ptr(scales)):
        raise ValueError("oracle_quantize_e4m3_columns failed")
    return codes, scales


def dequantize_e4m3(codes, scales, lib=None) -> np.ndarray:
    """scale[n] * e4m3(code[k][n]) in fp64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    K, N = codes.shape
    if scales.shape != (N,):
        raise ValueError("one scale per column")
    out = np.empty((K, N), dtype=np.float64)
    if (lib or _load()).oracle_dequantize_e4m3_columns(_ptr(codes), _ptr(scales), K, N,
                                                       _ptr(out)):
        raise ValueError("oracle_dequantize_e4m3_columns failed")
    return out


def e2m1_to_double(code: int, lib=None) -> float:
    return (lib or _load()).oracle_e2m1_to_double(int(code))


def e2m1_from_double(v: float, lib=None) -> int:
    """Nearest E2M1 code (ties to even, saturating at 6)."""
    return (lib or _load()).oracle_e2m1_from_double(float(v))


def mx_shared_exponent(amax: float, lib=None) -> int:
    return (lib or _load()).oracle_mx_shared_exponent(float(amax))


def quantize_mxfp4(w, lib=None):
    """MXFP4 quantisation of a K x N bf16 matrix along K: returns (codes
    uint8 K x N, one E2M1 code each; scales uint8 ceil(K/32) x N, E8M0)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    K, N = w.shape
    codes = np.empty((K, N), dtype=np.uint8)
    scales = np.empty(((K + 31) // 32, N), dtype=np.uint8)
    if (lib or _load()).oracle_quantize_mxfp4_columns(_ptr(w), K, N, _ptr(codes), _ptr(scales)):
        raise ValueError("oracle_quantize_mxfp4_columns failed")
    return codes, scales


def dequantize_mxfp4(codes, scales, lib=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K, N = codes.shape
    if scales.shape != ((K + 31) // 32, N):
        raise ValueError("one scale per 32-row block and column")
    out = np.empty((K, N), dtype=np.float64)
    if (lib or _load()).oracle_dequantize_mxfp4_columns(_ptr(codes), _ptr(scales), K, N,
                                                        _ptr(out)):
        raise ValueError("oracle_dequantize_mxfp4_columns failed")
    return out


def swiglu_fp8w(x, qg, sg, qu, su, rows=None, nthreads=0, lib=None):
    """silu(x.Wg) * (x.Wu) with Wg, Wu given as E4M3 codes and column scales
    (x in bf16 bits): the fp64 product of x and the dequantised weights."""
    return swiglu(bf16_array_to_double(x, lib), dequantize_e4m3(qg, sg, lib),
                  dequantize_e4m3(qu, su, lib), rows=rows, nthreads=nthreads, lib=lib)


def mlp_fp8w(x, qg, sg, qu, su, qd, sd, rows=None, nthreads=0, lib=None):
    """The full MLP with all three weights given as E4M3 codes and scales."""
    return mlp(bf16_array_to_double(x, lib), dequantize_e4m3(qg, sg, lib),
               dequantize_e4m3(qu, su, lib), dequantize_e4m3(qd, sd, lib), rows=rows,
               nthreads=nthreads, lib=lib)


def to_double(a, lib=None) -> np.ndarray:
    """Exact fp64 copy of a storage array (float32, float64, or bf16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return bf16_array_to_double(a, lib)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError("float32, float64 or bf16 bits expected")


def rmsnorm(r, gamma, eps, lib=None) -> np.ndarray:
    """n = r / sqrt(mean(r^2) + eps) * gamma per row, in fp64."""
    r = np.ascontiguousarray(r)
    gamma = np.ascontiguousarray(gamma)
    if _dtype_of(gamma) != _dtype_of(r):
        raise TypeError("r and gamma must share one dtype")
    M, d = r.shape
    if gamma.shape != (d,):
        raise ValueError("gamma must hold d values")
    out = np.empty((M, d), dtype=np.float64)
    rc = (lib or _load()).oracle_rmsnorm_rows(_dtype_of(r), _ptr(r), _ptr(gamma), float(eps), M, d,
                                              _ptr(out))
    if rc != 0:
        raise ValueError("oracle_rmsnorm_rows failed")
    return out


def mlp_block(r, gamma, eps, wg, wu, wd, bias=None, rows=None, nthreads=0, lib=None):
    """The MLP half of a pre-normalised layer ("Anatomie d'un transformeur
    sur GPU" §1.1; kernels 7 to 11 of §1.6): out = r + MLP(rmsnorm(r)) (+ bias
    on the down product, the Affine operation of "Où part le temps d'un
    token").  Weights are storage arrays or fp64 (dequantised) arrays; the
    normalised rows are not rounded.  fp64."""
    n = rmsnorm(r, gamma, eps, lib=lib)
    f = lambda a: to_double(a, lib)
    y = mlp(n, f(wg), f(wu), f(wd), rows=rows, nthreads=nthreads, lib=lib)
    if bias is not None:
        y = y + f(bias)[None, :]
    rr = f(r) if rows is None else f(r)[np.asarray(rows)]
    return rr + y


def default_threads() -> int:
    return _load().oracle_default_threads()


def lib_path() -> str:
    return _LIB


def load_library(path: str):
    """Bind another build of oracle.c (used by the tests that plant
    mistakes in a copy of the source); pass the handle as `lib=`."""
    return _bind(ctypes.CDLL(path))


def available_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
