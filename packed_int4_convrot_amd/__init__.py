"""Python binding of libck, the MI355X ConvRot packed-INT4 linear.

Argument marshalling only: tensors are checked for dtype, device and layout,
their pointers and strides are handed to the C ABI (include/ck.h) together with
torch's current HIP stream, and a status other than CK_OK becomes an exception
(ValueError for invalid arguments, RuntimeError otherwise).  Every step of the
computation runs in the HIP kernels of libck.so; there is no other code path.
Importing this package fails if libck.so has not been built
(``python -m packed_int4_convrot_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libck.so")

CK_OK, CK_ERR_INVALID_ARG, CK_ERR_UNSUPPORTED, CK_ERR_WORKSPACE, CK_ERR_HIP = range(5)
CK_WS_PER_CHANNEL, CK_WS_PER_GROUP = 0, 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

SIGNATURES = {
    "ck_status_str": ([_i32], ctypes.c_char_p),
    "ck_last_error_msg": ([], ctypes.c_char_p),
    "ck_version": ([], ctypes.c_char_p),
    "ck_rotate_quant": ([_p, _i64, _i64, _i64, _i32, _i32, _p, _i64, _p, _p], ctypes.c_int),
    "ck_w4_gemm_q": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i32, _i32, _i64, _p, _p, _i64, _p],
                     ctypes.c_int),
    "ck_w4_gemv": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i32, _i32, _i64, _p, _p, _i64, _p],
                   ctypes.c_int),
    "ck_linear_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "ck_w4a8_linear": ([_p, _i64, _i64, _i64, _i32, _p, _i64, _p, _i32, _i32, _i64, _p, _f32, _p,
                        _i64, _p, _sz, _p], ctypes.c_int),
    "ck_w4a4_linear": ([_p, _i64, _i64, _i64, _i32, _p, _i64, _p, _i32, _i32, _i64, _p, _f32, _p,
                        _i64, _p, _sz, _p], ctypes.c_int),
    "ck_w4a4_linear_noalloc": ([_p, _i64, _i64, _i64, _i32, _p, _i64, _p, _i32, _i32, _i64, _p, _f32, _p,
                                _i64, _p], ctypes.c_int),
    "ck_w4a16_gemv": ([_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i32, _i64, _p, _p, _i64, _p],
                      ctypes.c_int),
    "ck_w4a16_gemm": ([_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i32, _i64, _p, _p, _i64, _p],
                      ctypes.c_int),
    "ck_quantize_weights": ([_p, _i64, _i64, _i64, _i32, _i32, _p, _i64, _p, _p], ctypes.c_int),
    "ck_test_rotate_f32": ([_p, _i64, _i64, _i64, _i32, _p, _i64, _p], ctypes.c_int),
    "ck_test_gemm_i32": ([_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "ck_rotate_quant_packed4": ([_p, _i64, _i64, _i64, _i32, _p, _i64, _p, _p], ctypes.c_int),
    "ck_w4a4_gemm_packed": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i32, _i32, _i64, _p, _p, _i64, _p],
                            ctypes.c_int),
    "ck_test_gemm_i32_a4": ([_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "ck_test_linear_mfma_one_launch": ([_i32, _p, _i64, _i64, _i64, _i32, _p, _i64, _p, _i32, _i32, _i64, _p,
                                        _f32, _p, _i64, _p], ctypes.c_int),
}


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libck.so is not built (expected at %s); run `python -m packed_int4_convrot_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load_library()


class CKError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (lib.ck_status_str(status).decode(), msg))
        self.status = status


class CKInvalidArgument(CKError, ValueError):
    pass


def last_error() -> str:
    return lib.ck_last_error_msg().decode()


def version() -> str:
    return lib.ck_version().decode()


def _check(status: int):
    if status == CK_OK:
        return
    if status == CK_ERR_INVALID_ARG:
        raise CKInvalidArgument(status, last_error())
    raise CKError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _matrix(t, name, dtypes):
    """A 2-D GPU tensor of one of `dtypes` whose rows are disjoint runs of unit-stride
    elements (the layout the C ABI describes with one row stride)."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError("%s must be a 2-D tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit column stride" % name)
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        # expanded (stride 0) or overlapping rows: the C ABI would take them as
        # disjoint rows of stride >= K and touch memory past the tensor's storage
        raise ValueError("%s has row stride %d below its row length %d (expanded or overlapping rows)"
                         % (name, t.stride(0), t.shape[1]))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    return t


def _ld(t):
    """Row stride in elements.  A single row may report any stride, so it counts as its
    own length; for more rows _matrix has checked that the stride covers a row."""
    if t.shape[0] <= 1:
        return max(t.stride(0), t.shape[1])
    if t.stride(0) < t.shape[1]:
        raise ValueError("row stride %d below the row length %d" % (t.stride(0), t.shape[1]))
    return t.stride(0)


def _same_device(ref, *named):
    for name, t in named:
        if t is not None and t.device != ref.device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, ref.device))


def _dense(t, name, dtype, shape):
    """A contiguous tensor of exactly this shape and dtype on the GPU (the kernels index
    it as a packed array)."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be a %s tensor of shape %s" % (name, dtype, tuple(shape)))
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous GPU tensor" % name)
    return t


def _out(t, name, dtype, M, N):
    """An output matrix of M rows of N elements (row stride may exceed N)."""
    _matrix(t, name, (dtype,))
    if tuple(t.shape) != (M, N):
        raise ValueError("%s has shape %s, expected (%d, %d)" % (name, tuple(t.shape), M, N))
    return t


def _weights(packed, w_scales, per_group, K):
    _matrix(packed, "packed", (torch.uint8, torch.int8))
    if packed.shape[1] != K // 2:
        raise ValueError("packed has %d bytes per row, expected K/2 = %d" % (packed.shape[1], K // 2))
    N = packed.shape[0]
    if w_scales is not None:
        _dense(w_scales, "weight scales", torch.bfloat16, (K // 64, N) if per_group else (N,))
    return N


def workspace_bytes(M: int, K: int, N: int) -> int:
    """Workspace bytes of the whole-linear entry points for M rows, K columns, N outputs."""
    return int(lib.ck_linear_workspace_bytes(M, K, N))


def rotate_quant(x, G: int, bits: int, codes=None, row_scales=None):
    """codes int8 [M, K] and fp32 row scales [M] of a bf16 [M, K] (possibly strided) input."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if row_scales is None:
        row_scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _out(codes, "codes", torch.int8, M, K)
    _dense(row_scales, "row_scales", torch.float32, (M,))
    _same_device(x, ("codes", codes), ("row_scales", row_scales))
    _check(lib.ck_rotate_quant(_ptr(x), M, K, _ld(x), G, bits, _ptr(codes), _ld(codes),
                               _ptr(row_scales), _stream(x)))
    return codes, row_scales


def quantize_weights(w, G: int, per_group: bool, packed=None, scales=None):
    """Packed uint4 weights uint8 [N, K/2] and bf16 scales ([N] or [K/64, N]) of a
    bf16 weight [N, K] rotated by H_G: the producer of the matmuls' weight format."""
    _matrix(w, "w", (torch.bfloat16,))
    N, K = w.shape
    if packed is None:
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        shape = (K // 64, N) if per_group else (N,)
        scales = torch.empty(shape, dtype=torch.bfloat16, device=w.device)
    _out(packed, "packed", torch.uint8, N, K // 2)
    _dense(scales, "scales", torch.bfloat16, (K // 64, N) if per_group else (N,))
    _same_device(w, ("packed", packed), ("scales", scales))
    _check(lib.ck_quantize_weights(_ptr(w), N, K, _ld(w), G, 1 if per_group else 0, _ptr(packed),
                                   _ld(packed), _ptr(scales), _stream(w)))
    return packed, scales


def rotated_f32(x, G: int):
    """Rotated rows as the rotate-quant kernel holds them (divided by sqrt(G)), fp32 [M, K]."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    xr = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _check(lib.ck_test_rotate_f32(_ptr(x), M, K, _ld(x), G, _ptr(xr), _ld(xr), _stream(x)))
    return xr


def gemm_q(codes, row_scales, packed, w_scales, per_group: bool, bias=None, out=None,
           gemv: bool = False):
    """bf16 [M, N] matmul + scale epilogue on already quantised activations."""
    _matrix(codes, "codes", (torch.int8,))
    M, K = codes.shape
    N = _weights(packed, w_scales, per_group, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=codes.device)
    _dense(row_scales, "row_scales", torch.float32, (M,))
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    _out(out, "out", torch.bfloat16, M, N)
    _same_device(codes, ("row_scales", row_scales), ("packed", packed), ("w_scales", w_scales),
                 ("bias", bias), ("out", out))
    fn = lib.ck_w4_gemv if gemv else lib.ck_w4_gemm_q
    _check(fn(_ptr(codes), _ld(codes), _ptr(row_scales), M, K, _ptr(packed), _ld(packed),
              _ptr(w_scales), CK_WS_PER_GROUP if per_group else CK_WS_PER_CHANNEL, 64, N,
              _ptr(bias), _ptr(out), _ld(out), _stream(codes)))
    return out


def gemv(codes, row_scales, packed, w_scales, per_group: bool, bias=None, out=None):
    """Decode form of gemm_q (1 <= M <= 8)."""
    return gemm_q(codes, row_scales, packed, w_scales, per_group, bias, out, gemv=True)


def linear(x, G: int, bits: int, packed, w_scales, per_group: bool, bias=None,
           x_scale: float = 1.0, out=None, workspace=None):
    """Whole ConvRot linear: bf16 [M, N] = rotate-quant(x) @ W4^T with the scale epilogue."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    N = _weights(packed, w_scales, per_group, K)
    if bits not in (8, 4):
        raise ValueError("bits must be 8 or 4")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    need = workspace_bytes(M, K, N)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    _out(out, "out", torch.bfloat16, M, N)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    _same_device(x, ("packed", packed), ("w_scales", w_scales), ("bias", bias), ("out", out),
                 ("workspace", workspace))
    fn = lib.ck_w4a8_linear if bits == 8 else lib.ck_w4a4_linear
    _check(fn(_ptr(x), M, K, _ld(x), G, _ptr(packed), _ld(packed), _ptr(w_scales),
              CK_WS_PER_GROUP if per_group else CK_WS_PER_CHANNEL, 64, N, _ptr(bias), x_scale,
              _ptr(out), _ld(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream(x)))
    return out


def linear_mfma_one_launch(x, G: int, bits: int, packed, w_scales, per_group: bool, bias=None,
                                x_scale: float = 1.0, out=None):
    """ck_test_linear_mfma_one_launch: the whole linear forced onto its one-launch
    MFMA kernel (1 <= M <= 8, K <= 4096, any N), for testing its launch shapes."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    N = _weights(packed, w_scales, per_group, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    _out(out, "out", torch.bfloat16, M, N)
    _same_device(x, ("packed", packed), ("w_scales", w_scales), ("bias", bias), ("out", out))
    _check(lib.ck_test_linear_mfma_one_launch(bits, _ptr(x), M, K, _ld(x), G, _ptr(packed), _ld(packed),
                                              _ptr(w_scales), CK_WS_PER_GROUP if per_group else CK_WS_PER_CHANNEL,
                                              64, N, _ptr(bias), x_scale, _ptr(out), _ld(out), _stream(x)))
    return out


NOALLOC_SCRATCH_BYTES = (64 << 20) + (64 << 10)   # the library's static scratch per GPU (include/ck.h)


def w4a4_linear_noalloc(x, G: int, packed, w_scales, per_group: bool, bias=None,
                        x_scale: float = 1.0, out=None):
    """ck_w4a4_linear without a workspace: the codes live in the library's static
    scratch (one per GPU, shared by every call on it; calls must not overlap)."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    N = _weights(packed, w_scales, per_group, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    _out(out, "out", torch.bfloat16, M, N)
    _same_device(x, ("packed", packed), ("w_scales", w_scales), ("bias", bias), ("out", out))
    _check(lib.ck_w4a4_linear_noalloc(_ptr(x), M, K, _ld(x), G, _ptr(packed), _ld(packed), _ptr(w_scales),
                                      CK_WS_PER_GROUP if per_group else CK_WS_PER_CHANNEL, 64, N, _ptr(bias),
                                      x_scale, _ptr(out), _ld(out), _stream(x)))
    return out


def w4a8_linear(x, G, packed, w_scales, per_group, **kw):
    return linear(x, G, 8, packed, w_scales, per_group, **kw)


def w4a4_linear(x, G, packed, w_scales, per_group, **kw):
    return linear(x, G, 4, packed, w_scales, per_group, **kw)


def w4a16_gemm(x, packed, scales, zeros, bias=None, out=None):
    """AWQ W4A16 product for any M on the dequantise path (W rebuilt in bf16), bf16 [M, N]."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    N = _weights(packed, scales, True, K)
    _dense(zeros, "zeros", torch.bfloat16, (K // 64, N))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    _out(out, "out", torch.bfloat16, M, N)
    _same_device(x, ("packed", packed), ("scales", scales), ("zeros", zeros), ("bias", bias),
                 ("out", out))
    _check(lib.ck_w4a16_gemm(_ptr(x), M, K, _ld(x), _ptr(packed), _ld(packed), _ptr(scales),
                             _ptr(zeros), 64, N, _ptr(bias), _ptr(out), _ld(out), _stream(x)))
    return out


def w4a16_gemv(x, packed, scales, zeros, bias=None, out=None):
    """AWQ W4A16 product, bf16 [M, N] (1 <= M <= 8)."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    N = _weights(packed, scales, True, K)
    _dense(zeros, "zeros", torch.bfloat16, (K // 64, N))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    _out(out, "out", torch.bfloat16, M, N)
    _same_device(x, ("packed", packed), ("scales", scales), ("zeros", zeros), ("bias", bias),
                 ("out", out))
    _check(lib.ck_w4a16_gemv(_ptr(x), M, K, _ld(x), _ptr(packed), _ld(packed), _ptr(scales),
                             _ptr(zeros), 64, N, _ptr(bias), _ptr(out), _ld(out), _stream(x)))
    return out


def rotate_quant_packed4(x, G: int, codes4=None, row_scales=None):
    """W4A4 codes packed two per byte, uint8 [M, K/2] (column 2j in the low
    nibble, 4-bit two's complement), and fp32 row scales [M]."""
    _matrix(x, "x", (torch.bfloat16,))
    M, K = x.shape
    if codes4 is None:
        codes4 = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if row_scales is None:
        row_scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _out(codes4, "codes4", torch.uint8, M, K // 2)
    _dense(row_scales, "row_scales", torch.float32, (M,))
    _same_device(x, ("codes4", codes4), ("row_scales", row_scales))
    _check(lib.ck_rotate_quant_packed4(_ptr(x), M, K, _ld(x), G, _ptr(codes4), _ld(codes4),
                                       _ptr(row_scales), _stream(x)))
    return codes4, row_scales


def gemm_packed4(codes4, row_scales, packed, w_scales, per_group: bool, bias=None, out=None):
    """bf16 [M, N] linear output from packed W4A4 codes (rotate_quant_packed4) on the tiled GEMM."""
    _matrix(codes4, "codes4", (torch.uint8,))
    M = codes4.shape[0]
    K = 2 * codes4.shape[1]
    N = _weights(packed, w_scales, per_group, K)
    _dense(row_scales, "row_scales", torch.float32, (M,))
    if bias is not None:
        _dense(bias, "bias", torch.bfloat16, (N,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=codes4.device)
    _out(out, "out", torch.bfloat16, M, N)
    _same_device(codes4, ("row_scales", row_scales), ("packed", packed), ("w_scales", w_scales),
                 ("bias", bias), ("out", out))
    _check(lib.ck_w4a4_gemm_packed(_ptr(codes4), _ld(codes4), _ptr(row_scales), M, K, _ptr(packed),
                                   _ld(packed), _ptr(w_scales), 1 if per_group else 0, 64, N, _ptr(bias),
                                   _ptr(out), _ld(out), _stream(codes4)))
    return out


def accumulators_i32_a4(codes4, K: int, packed):
    """int32 [M, N] accumulators of the tiled GEMM on packed W4A4 codes uint8 [M, K/2]."""
    _matrix(codes4, "codes4", (torch.uint8,))
    M = codes4.shape[0]
    if codes4.shape[1] != K // 2:
        raise ValueError("codes4 must have K/2 = %d columns (got %d)" % (K // 2, codes4.shape[1]))
    N = _weights(packed, None, False, K)
    acc = torch.empty((M, N), dtype=torch.int32, device=codes4.device)
    _same_device(codes4, ("packed", packed))
    _check(lib.ck_test_gemm_i32_a4(_ptr(codes4), _ld(codes4), M, K, _ptr(packed), _ld(packed), N,
                                   _ptr(acc), _ld(acc), _stream(codes4)))
    return acc


def accumulators_i32(codes, packed):
    """int32 [M, N] accumulators sum_k codes[m,k] * (q[n,k] - 8) from the matmul kernels."""
    _matrix(codes, "codes", (torch.int8,))
    M, K = codes.shape
    N = _weights(packed, None, False, K)
    acc = torch.empty((M, N), dtype=torch.int32, device=codes.device)
    _check(lib.ck_test_gemm_i32(_ptr(codes), _ld(codes), M, K, _ptr(packed), _ld(packed), N,
                                _ptr(acc), _ld(acc), _stream(codes)))
    return acc
