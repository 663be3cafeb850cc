"""Reference oracle for the ConvRot packed-INT4 linear (CPU, fp64).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this package; the library in
``packed_int4_convrot_amd/`` never does.  The arithmetic lives in
``oracle.c`` (plain single-threaded C, compiled with -ffp-contract=off); this
module only builds it, marshals numpy arrays and chains its steps in the
order the pages give them:

  rotate (x . H_G / sqrt(G), per contiguous group)  -> quantize (rowwise
  absmax, fp32 decision) -> unpack (q - 8) -> exact integer matmul ->
  scale epilogue (fp64)

and, for the weights, rotate -> quantize_weights (absmax/7 per row or per
64-column group, bf16 scale, fp32 decision) -> pack.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, library routines and the worked examples in ``tests/golden/``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

QMAX = {8: 127, 4: 7}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
             "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        sig = {
            "oracle_hadamard": [i64, p],
            "oracle_rotate": [p, i64, i64, i64, i64, p, i64],
            "oracle_quantize": [p, i64, i64, i64, i32, p, i64, p],
            "oracle_unpack": [p, i64, i64, i64, p],
            "oracle_int_gemm": [p, i64, i64, i64, p, i64, i64, p],
            "oracle_epilogue": [p, i64, i64, i64, p, p, i32, p, ctypes.c_double, p],
            "oracle_awq_gemv": [p, i64, i64, i64, p, i64, p, p, i64, i64, p, p],
            "oracle_quantize_weights": [p, i64, i64, i64, i32, p, i64, p],
            "oracle_awq_dequantize": [p, i64, i64, i64, p, p, i64, p],
            "oracle_bf16_matmul": [p, i64, i64, i64, p, i64, i64, p, p],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def _u16(a) -> np.ndarray:
    """Accept bf16 bit patterns as a numpy uint16/int16 array or a torch bf16 tensor."""
    if hasattr(a, "view") and hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.contiguous().view(torch.int16).numpy()
    a = np.asarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("bf16 data must be given as uint16 bit patterns")
    return np.ascontiguousarray(a)


def hadamard(G: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_G (int8, entries +-1, natural order)."""
    H = np.empty((G, G), dtype=np.int8)
    _check(_load().oracle_hadamard(G, _ptr(H)), "hadamard")
    return H


def rotate(x, G: int, K: int | None = None) -> np.ndarray:
    """fp32 [M, K] rotated rows; x is bf16 [M, ldx] and the first K columns are used."""
    x = _u16(x)
    M, ldx = x.shape
    K = ldx if K is None else K
    xr = np.empty((M, K), dtype=np.float32)
    _check(_load().oracle_rotate(_ptr(x), M, K, ldx, G, _ptr(xr), K), "rotate")
    return xr


def quantize(xr: np.ndarray, bits: int):
    """(codes int8 [M, K], row scales fp32 [M]) from rotated fp32 rows."""
    xr = np.ascontiguousarray(xr, dtype=np.float32)
    M, K = xr.shape
    codes = np.empty((M, K), dtype=np.int8)
    scales = np.empty((M,), dtype=np.float32)
    _check(_load().oracle_quantize(_ptr(xr), M, K, K, QMAX[bits], _ptr(codes), K, _ptr(scales)),
           "quantize")
    return codes, scales


def rotate_quant(x, G: int, bits: int, K: int | None = None):
    """Rotation followed by rowwise quantisation: (codes, scales)."""
    return quantize(rotate(x, G, K), bits)


def quantize_weights(wr: np.ndarray, per_group: bool, Gw: int = 64):
    """(packed uint8 [N, K/2], bf16 scale bits uint16 [N] or [K/Gw, N]) from rotated
    fp32 weight rows: symmetric absmax/7 codes, stored as q = code + 8."""
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    N, K = wr.shape
    packed = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((K // Gw, N) if per_group else (N,), dtype=np.uint16)
    _check(_load().oracle_quantize_weights(_ptr(wr), N, K, K, Gw if per_group else 0, _ptr(packed),
                                           K // 2, _ptr(scales)), "quantize_weights")
    return packed, scales


def rotate_quantize_weights(w, G: int, per_group: bool, Gw: int = 64):
    """The offline weight producer: rotation by H_G, then quantize_weights."""
    return quantize_weights(rotate(w, G), per_group, Gw)


def unpack(packed, K: int | None = None) -> np.ndarray:
    """int8 [N, K] weight values q - 8 from packed uint8 [N, ldw]."""
    packed = np.ascontiguousarray(np.asarray(packed).view(np.uint8))
    N, ldw = packed.shape
    K = 2 * ldw if K is None else K
    w = np.empty((N, K), dtype=np.int8)
    _check(_load().oracle_unpack(_ptr(packed), N, K, ldw, _ptr(w)), "unpack")
    return w


def int_gemm(codes: np.ndarray, w: np.ndarray, group: int | None = None) -> np.ndarray:
    """Exact sums of codes[m,k] * w[n,k]: int64 [M, N] (group None) or [M, N, K/group]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    M, K = codes.shape
    N = w.shape[0]
    Gk = K if group is None else group
    acc = np.empty((M, N, K // Gk), dtype=np.int64)
    _check(_load().oracle_int_gemm(_ptr(codes), K, M, K, _ptr(w), N, Gk, _ptr(acc)), "int_gemm")
    return acc[:, :, 0] if group is None else acc


def epilogue(acc: np.ndarray, row_scales, w_scales, per_group: bool, bias=None,
             x_scale: float = 1.0) -> np.ndarray:
    """fp64 [M, N] output from exact accumulators and the activation / weight scales;
    x_scale > 0 is the input scale (the linear of x_scale * x: the row scale times
    x_scale, the bias unscaled)."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    M, N = acc.shape[:2]
    ng = acc.shape[2] if acc.ndim == 3 else 1
    rs = np.ascontiguousarray(row_scales, dtype=np.float32)
    ws = _u16(w_scales)
    b = None if bias is None else _u16(bias)
    out = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_epilogue(_ptr(acc), M, N, ng, _ptr(rs), _ptr(ws), 1 if per_group else 0,
                                   _ptr(b), float(x_scale), _ptr(out)), "epilogue")
    return out


def gemm_q(codes, row_scales, packed, w_scales, per_group: bool, Gw: int = 64, bias=None,
           x_scale: float = 1.0):
    """fp64 linear output from given activation codes and scales (the matmul half)."""
    w = unpack(packed, codes.shape[1])
    acc = int_gemm(codes, w, Gw if per_group else None)
    return epilogue(acc, row_scales, w_scales, per_group, bias, x_scale)


def linear(x, G: int, bits: int, packed, w_scales, per_group: bool, Gw: int = 64, bias=None,
           K: int | None = None, x_scale: float = 1.0):
    """Whole ConvRot linear of x_scale * x: returns (out fp64 [M,N], codes, row scales).
    The codes and row scales returned are those of x itself."""
    codes, scales = rotate_quant(x, G, bits, K)
    return gemm_q(codes, scales, packed, w_scales, per_group, Gw, bias, x_scale), codes, scales


def awq_gemv(x, packed, scales, zeros, Gw: int = 64, bias=None, K: int | None = None) -> np.ndarray:
    """fp64 [M, N] AWQ W4A16 product with the weights dequantised in fp64."""
    x = _u16(x)
    M, ldx = x.shape
    K = ldx if K is None else K
    packed = np.ascontiguousarray(np.asarray(packed).view(np.uint8))
    N, ldw = packed.shape
    s = _u16(scales)
    z = _u16(zeros)
    b = None if bias is None else _u16(bias)
    out = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_awq_gemv(_ptr(x), M, K, ldx, _ptr(packed), ldw, _ptr(s), _ptr(z), Gw, N,
                                   _ptr(b), _ptr(out)), "awq_gemv")
    return out


def awq_dequantize(packed, scales, zeros, Gw: int = 64, K: int | None = None) -> np.ndarray:
    """bf16 bits [N, K]: the AWQ weight rebuilt as the page's dequantize() does (each
    tensor operation rounded to bf16)."""
    packed = np.ascontiguousarray(np.asarray(packed).view(np.uint8))
    N, ldw = packed.shape
    K = 2 * ldw if K is None else K
    s = _u16(scales)
    z = _u16(zeros)
    w = np.empty((N, K), dtype=np.uint16)
    _check(_load().oracle_awq_dequantize(_ptr(packed), N, K, ldw, _ptr(s), _ptr(z), Gw, _ptr(w)),
           "awq_dequantize")
    return w


def bf16_matmul(x, w, bias=None) -> np.ndarray:
    """fp64 [M, N] = x . w^T (+ bias) for bf16 x [M, K] and w [N, K]."""
    x = _u16(x)
    w = _u16(w)
    M, K = x.shape
    N = w.shape[0]
    b = None if bias is None else _u16(bias)
    out = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_bf16_matmul(_ptr(x), M, K, K, _ptr(w), N, w.shape[1], _ptr(b), _ptr(out)),
           "bf16_matmul")
    return out


def awq_gemm(x, packed, scales, zeros, Gw: int = 64, bias=None) -> np.ndarray:
    """fp64 [M, N] AWQ product on the dequantised bf16 weight (the prefill path)."""
    x = _u16(x)
    return bf16_matmul(x, awq_dequantize(packed, scales, zeros, Gw, x.shape[1]), bias)
