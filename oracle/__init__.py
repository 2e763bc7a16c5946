"""CPU oracle for the planned dense GEMM - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product.

The arithmetic lives in ``oracle.c`` (plain C, binary64 / int64, k ascending);
this module only marshals numpy arrays.  Page citations: see the header of
``oracle.c``.  Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` against exact rational brute force, exhaustive
codec checks, closed forms and invariants.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

KIND = {"f16": 0, "bf16": 1, "f32": 2, "i8": 3, "i32": 4, "e2m1": 5}
_NP = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i8": np.int8,
       "i32": np.int32, "e2m1": np.uint8}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = C.CDLL(_build.LIB)
    p, i64, i32, d = C.c_void_p, C.c_int64, C.c_int, C.c_double
    lib.orc_gemm_real.argtypes = [i64, i64, i64, i32, p, i32, p, p, i64, d, d, i32, p,
                                  i32, p, i32, p, i32]
    lib.orc_gemm_real.restype = i32
    lib.orc_gemm_int.argtypes = [i64, i64, i64, p, p, i64, i64, p, p, p, i32]
    lib.orc_gemm_int.restype = i64
    lib.orc_requant.argtypes = [i64, i64, p, C.c_float, p, i32, p]
    lib.orc_requant.restype = i32
    lib.orc_gemm_mx.argtypes = [i64, i64, i64, p, p, p, p, d, i32, p, i32, p, i32]
    lib.orc_gemm_mx.restype = i32
    lib.orc_quant_mx_e4m3.argtypes = [i64, i64, p, p, p]
    lib.orc_quant_mx_e4m3.restype = i32
    for name in ("orc_f16_values", "orc_bf16_values", "orc_e2m1_values", "orc_fp8e4m3_values",
                 "orc_e8m0_values", "orc_fp8e4m3_rne_sat_array",
                 "orc_f16_rne_array", "orc_bf16_rne_array", "orc_gelu_erf_array"):
        getattr(lib, name).argtypes = [i64, p, p]
        getattr(lib, name).restype = None
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, kind):
    """Contiguous numpy view with the storage type of ``kind`` (bit patterns)."""
    a = np.ascontiguousarray(a)
    want = _NP[kind]
    if a.dtype != want:
        if a.dtype.itemsize != np.dtype(want).itemsize:
            raise TypeError(f"array of {a.dtype} cannot hold {kind} elements")
        a = a.view(want)
    return a


def max_threads() -> int:
    return int(_load().orc_max_threads())


# ------------------------------------------------------------------ codecs
def f16_values(bits) -> np.ndarray:
    b = _c(bits, "f16")
    out = np.empty(b.shape, np.float64)
    _load().orc_f16_values(b.size, _ptr(b), _ptr(out))
    return out


def bf16_values(bits) -> np.ndarray:
    b = _c(bits, "bf16")
    out = np.empty(b.shape, np.float64)
    _load().orc_bf16_values(b.size, _ptr(b), _ptr(out))
    return out


def e2m1_values(codes) -> np.ndarray:
    c = _c(codes, "e2m1")
    out = np.empty(c.shape, np.float64)
    _load().orc_e2m1_values(c.size, _ptr(c), _ptr(out))
    return out


def fp8e4m3_values(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_fp8e4m3_values(c.size, _ptr(c), _ptr(out))
    return out


def e8m0_values(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e8m0_values(c.size, _ptr(c), _ptr(out))
    return out


def fp8e4m3_rne_sat(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    _load().orc_fp8e4m3_rne_sat_array(x.size, _ptr(x), _ptr(out))
    return out


def f16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f16_rne_array(x.size, _ptr(x), _ptr(out))
    return out


def bf16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().orc_bf16_rne_array(x.size, _ptr(x), _ptr(out))
    return out


def gelu_erf(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.float64)
    _load().orc_gelu_erf_array(x.size, _ptr(x), _ptr(out))
    return out


def values(bits, kind) -> np.ndarray:
    """Decode stored elements of ``kind`` to binary64."""
    if kind == "f16":
        return f16_values(bits)
    if kind == "bf16":
        return bf16_values(bits)
    if kind == "e2m1":
        return e2m1_values(bits)
    return np.asarray(bits).astype(np.float64)


def rne(x, kind) -> np.ndarray:
    """Round binary64 values to ``kind`` (f16 / bf16 bits, or f32 values)."""
    if kind == "f16":
        return f16_rne(x)
    if kind == "bf16":
        return bf16_rne(x)
    if kind == "f32":
        return np.asarray(x, np.float64).astype(np.float32)
    raise ValueError(kind)


# -------------------------------------------------------------------- GEMMs
def gemm_real(A, B, *, a_kind, b_kind, scale=None, group_k=32, alpha=1.0, beta=0.0,
              D=None, d_kind="f16", bias=None, bias_kind="f16", act=0, nthreads=0):
    """r = act(alpha * A.B + beta * D + bias) in binary64, unrounded.

    A: M x K stored elements of ``a_kind``; B: K x N of ``b_kind`` (for e2m1 one
    code per element, logical [K][N]); scale: binary16 bits [K/group_k][N]
    (e2m1 only); D: M x N of ``d_kind``; bias: [N] of ``bias_kind``;
    act: 0 identity, 1 GELU (erf form).
    """
    A = _c(A, a_kind)
    B = _c(B, b_kind)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    sc = _c(scale, "f16") if scale is not None else None
    Dc = _c(D, d_kind) if D is not None else None
    bc = _c(bias, bias_kind) if bias is not None else None
    R = np.empty((M, N), np.float64)
    rc = _load().orc_gemm_real(M, N, K, KIND[a_kind], _ptr(A), KIND[b_kind], _ptr(B),
                               _ptr(sc), int(group_k), float(alpha), float(beta),
                               KIND[d_kind], _ptr(Dc), KIND[bias_kind], _ptr(bc),
                               int(act), _ptr(R), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return R


def gemm_int(A, B, *, alpha=1, beta=0, D=None, nthreads=0):
    """Exact integer GEMM: returns (R int64, C int32 wrapped, n_overflow)."""
    A = _c(A, "i8")
    B = _c(B, "i8")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    Dc = _c(D, "i32") if D is not None else None
    R = np.empty((M, N), np.int64)
    Cw = np.empty((M, N), np.int32)
    ov = _load().orc_gemm_int(M, N, K, _ptr(A), _ptr(B), int(alpha), int(beta), _ptr(Dc),
                              _ptr(R), _ptr(Cw), int(nthreads))
    if ov < 0:
        raise ValueError("oracle rejected the arguments")
    return R, Cw, int(ov)


def gemm_mx(A, SA, B, SB, *, alpha=1.0, bias=None, bias_kind="f16", act=0, nthreads=0):
    """MX block-scaled GEMM in binary64, unrounded.

    A: fp8 e4m3 codes M x K; SA: e8m0 codes [M][K/32]; B: e2m1 codes, logical
    [K][N], one per byte; SB: e8m0 codes [K/32][N]; bias: [N] of ``bias_kind``;
    act: 0 identity, 1 GELU (erf form).
    """
    A = np.ascontiguousarray(A, np.uint8)
    SA = np.ascontiguousarray(SA, np.uint8)
    B = np.ascontiguousarray(B, np.uint8)
    SB = np.ascontiguousarray(SB, np.uint8)
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or SA.shape != (M, K // 32) or SB.shape != (K // 32, N):
        raise ValueError("operand shapes disagree")
    bc = _c(bias, bias_kind) if bias is not None else None
    R = np.empty((M, N), np.float64)
    rc = _load().orc_gemm_mx(M, N, K, _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), float(alpha),
                             KIND[bias_kind], _ptr(bc), int(act), _ptr(R), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return R


def quant_mx(X):
    """binary16 bits M x K -> (fp8 e4m3 codes M x K, e8m0 scale codes [M][K/32])."""
    X = _c(X, "f16")
    M, K = X.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, K // 32), np.uint8)
    rc = _load().orc_quant_mx_e4m3(M, K, _ptr(X), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return codes, scales


def requant(acc, *, alpha, bias=None, out="i8"):
    """Requantise a 32-bit accumulator: binary32 steps, round to nearest even."""
    acc = _c(acc, "i32")
    M, N = acc.shape
    bc = None if bias is None else np.ascontiguousarray(bias, np.float32)
    res = np.empty((M, N), np.int8 if out == "i8" else np.uint16)
    rc = _load().orc_requant(M, N, _ptr(acc), float(alpha), _ptr(bc), KIND[out], _ptr(res))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return res
