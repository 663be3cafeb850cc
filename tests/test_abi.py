"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before anything is enqueued.

The fake device pointers below are never dereferenced: every call here fails
validation, which runs entirely on the host before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ck.h")

ck = pytest.importorskip("packed_int4_convrot_amd")
lib = ck.lib

P = 0x10000000  # 256-byte aligned fake device address (never dereferenced)
P2 = 0x20000000
P3 = 0x30000000
P4 = 0x40000000
P5 = 0x50000000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ck_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), "libck.so does not export %s" % n
        assert n in ck.SIGNATURES, "binding lacks a signature for %s" % n


def test_status_strings_and_version():
    assert lib.ck_status_str(0) == b"CK_OK"
    assert lib.ck_status_str(3) == b"CK_ERR_WORKSPACE"
    assert lib.ck_version().startswith(b"ck ")


def test_workspace_bytes():
    assert lib.ck_linear_workspace_bytes(0, 3840, 3840) == 0
    ws = lib.ck_linear_workspace_bytes(32, 3840, 3840)
    assert ws >= 32 * 3840 + 32 * 4 and ws % 256 == 0
    assert lib.ck_linear_workspace_bytes(8192, 10240, 3840) == 8192 * 10240 + 32768


def rq(x=P, M=4, K=256, ldx=256, G=64, bits=8, codes=P2, ldq=256, rs=P3):
    return lib.ck_rotate_quant(x, M, K, ldx, G, bits, codes, ldq, rs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(G=32), ck.CK_ERR_UNSUPPORTED),
    (dict(G=128), ck.CK_ERR_UNSUPPORTED),
    (dict(bits=6), ck.CK_ERR_UNSUPPORTED),
    (dict(K=0), ck.CK_ERR_INVALID_ARG),
    (dict(K=96, ldx=96, ldq=96), ck.CK_ERR_INVALID_ARG),         # K % 64
    (dict(K=320, ldx=320, ldq=320, G=256), ck.CK_ERR_INVALID_ARG),  # K % G
    (dict(K=65536, ldx=65536, ldq=65536), ck.CK_ERR_UNSUPPORTED),
    (dict(M=-1), ck.CK_ERR_INVALID_ARG),
    (dict(x=None), ck.CK_ERR_INVALID_ARG),
    (dict(codes=None), ck.CK_ERR_INVALID_ARG),
    (dict(rs=None), ck.CK_ERR_INVALID_ARG),
    (dict(ldx=200), ck.CK_ERR_INVALID_ARG),
    (dict(ldx=260), ck.CK_ERR_INVALID_ARG),      # not a multiple of 8
    (dict(ldq=264), ck.CK_ERR_INVALID_ARG),      # not a multiple of 16
    (dict(x=P + 8), ck.CK_ERR_INVALID_ARG),      # misaligned
    (dict(codes=P + 512), ck.CK_ERR_INVALID_ARG),  # overlaps x
])
def test_rotate_quant_rejects(kw, status):
    assert rq(**kw) == status
    assert lib.ck_last_error_msg() != b""


def test_zero_rows_is_noop():
    assert rq(M=0, x=None, codes=None, rs=None) == ck.CK_OK


def gq(fn=None, codes=P, ldq=256, rs=P2, M=4, K=256, packed=P3, ldw=128, ws=P4, kind=1, Gw=64,
       N=64, bias=None, out=P5, ldo=64):
    fn = fn or lib.ck_w4_gemm_q
    return fn(codes, ldq, rs, M, K, packed, ldw, ws, kind, Gw, N, bias, out, ldo, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=40), ck.CK_ERR_UNSUPPORTED),
    (dict(N=0), ck.CK_ERR_INVALID_ARG),
    (dict(Gw=128), ck.CK_ERR_UNSUPPORTED),
    (dict(kind=5), ck.CK_ERR_INVALID_ARG),
    (dict(ldw=100), ck.CK_ERR_INVALID_ARG),
    (dict(packed=P3 + 4), ck.CK_ERR_INVALID_ARG),
    (dict(ws=None), ck.CK_ERR_INVALID_ARG),
    (dict(out=None), ck.CK_ERR_INVALID_ARG),
    (dict(ldo=32), ck.CK_ERR_INVALID_ARG),
    (dict(ldo=68), ck.CK_ERR_INVALID_ARG),       # rows not 16-byte aligned
    (dict(out=P5 + 4), ck.CK_ERR_INVALID_ARG),   # output not 16-byte aligned
    (dict(out=P3), ck.CK_ERR_INVALID_ARG),       # overlaps the packed weights
    (dict(out=P + 128), ck.CK_ERR_INVALID_ARG),  # overlaps the codes
    (dict(rs=None), ck.CK_ERR_INVALID_ARG),
])
def test_gemm_q_rejects(kw, status):
    assert gq(**kw) == status


def test_per_group_scales_need_16_byte_alignment():
    # the decode kernels read a row block's per-group scales with 16-byte loads
    assert gq(ws=P4 + 8, kind=1) == ck.CK_ERR_INVALID_ARG
    assert b"16-byte" in lib.ck_last_error_msg()


def test_launch_size_limits():
    # rows beyond one launch's grid, and a tiled GEMM whose tile grid would overflow
    assert rq(M=(1 << 22) + 1) == ck.CK_ERR_UNSUPPORTED
    # 2^22 rows of 1024-thread workgroups (K above 16384) would be 2^32 work-items,
    # one more than a grid dimension holds
    assert rq(M=(1 << 22), K=16448, ldx=16448, ldq=16448) == ck.CK_ERR_UNSUPPORTED
    assert lib.ck_quantize_weights(P, 1 << 22, 16448, 16448, 64, 0, P2, 8224, P3, None) == ck.CK_ERR_UNSUPPORTED
    assert gq(M=(1 << 22) - 1, N=(1 << 22) - 16, ldo=(1 << 22) - 16) == ck.CK_ERR_UNSUPPORTED
    assert b"too large" in lib.ck_last_error_msg()
    assert gq(N=(1 << 22)) == ck.CK_ERR_UNSUPPORTED
    # row strides beyond 32-bit buffer offsets of a 256-row tile
    assert gq(ldq=(1 << 23) + 16) == ck.CK_ERR_UNSUPPORTED
    assert gq(ldw=(1 << 23) + 16) == ck.CK_ERR_UNSUPPORTED


def test_gemv_rejects_large_m():
    assert gq(fn=lib.ck_w4_gemv, M=9) == ck.CK_ERR_UNSUPPORTED
    assert gq(fn=lib.ck_w4_gemv, M=0) == ck.CK_OK


def lin(fn=None, x=P, M=4, K=256, ldx=256, G=64, packed=P3, ldw=128, ws_=P4, kind=0, Gw=64, N=64,
        bias=None, xs=1.0, out=P5, ldo=64, work=P2, wsb=1 << 20):
    fn = fn or lib.ck_w4a8_linear
    return fn(x, M, K, ldx, G, packed, ldw, ws_, kind, Gw, N, bias, xs, out, ldo, work, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(work=None), ck.CK_ERR_WORKSPACE),
    (dict(wsb=100), ck.CK_ERR_WORKSPACE),
    (dict(work=P2 + 16), ck.CK_ERR_WORKSPACE),   # not 256-byte aligned
    (dict(work=P), ck.CK_ERR_WORKSPACE),         # workspace overlaps x
    (dict(xs=0.0), ck.CK_ERR_INVALID_ARG),
    (dict(xs=float("inf")), ck.CK_ERR_INVALID_ARG),
    (dict(G=8), ck.CK_ERR_UNSUPPORTED),
    (dict(out=P2), ck.CK_ERR_INVALID_ARG),       # output overlaps the workspace
])
def test_linear_rejects(kw, status):
    assert lin(**kw) == status
    assert lin(fn=lib.ck_w4a4_linear, **kw) == status


def test_awq_rejects():
    f = lib.ck_w4a16_gemv
    assert f(P, 9, 256, 256, P3, 128, P4, P2, 64, 64, None, P5, 64, None) == ck.CK_ERR_UNSUPPORTED
    assert f(P, 1, 256, 256, P3, 128, P4, None, 64, 64, None, P5, 64, None) == ck.CK_ERR_INVALID_ARG
    assert f(P, 1, 256, 256, P3, 128, P4, P2, 32, 64, None, P5, 64, None) == ck.CK_ERR_UNSUPPORTED
    assert f(P, 1, 32768, 32768, P3, 16384, P4, P2, 64, 64, None, P5, 64, None) == ck.CK_ERR_UNSUPPORTED
    assert f(P, 1, 256, 256, P3, 128, P4 + 2, P2, 64, 64, None, P5, 64, None) == ck.CK_ERR_INVALID_ARG
    assert f(P, 1, 256, 256, P3, 128, P4, P2 + 8, 64, 64, None, P5, 64, None) == ck.CK_ERR_INVALID_ARG


def test_awq_gemm_rejects():
    f = lib.ck_w4a16_gemm
    args = [P, 300, 256, 256, P3, 128, P4, P2, 64, 64, None, P5, 64, None]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a7=None) == ck.CK_ERR_INVALID_ARG          # zeros
    assert call(a6=P4 + 2) == ck.CK_ERR_INVALID_ARG        # scales 16-byte aligned
    assert call(a7=P2 + 8) == ck.CK_ERR_INVALID_ARG        # zeros 16-byte aligned
    assert call(a8=32) == ck.CK_ERR_UNSUPPORTED             # Gw
    assert call(a9=40) == ck.CK_ERR_UNSUPPORTED             # N % 16
    assert call(a3=200) == ck.CK_ERR_INVALID_ARG            # ldx < K
    assert call(a3=(1 << 22) + 8) == ck.CK_ERR_UNSUPPORTED   # ldx beyond the buffer offsets
    assert call(a11=P + 64) == ck.CK_ERR_INVALID_ARG        # output overlaps x
    assert call(a12=68) == ck.CK_ERR_INVALID_ARG            # ldo % 8
    assert call(a1=0, a0=None, a11=None) == ck.CK_OK


def test_gemm_packed4_rejects():
    f = lib.ck_w4a4_gemm_packed
    ok = dict(c=P, ldq=128, rs=P2, M=4, K=256, w=P3, ldw=128, s=P4, kind=0, Gw=64, N=64, b=None, o=P5, ldo=64)
    def call(**kw):
        a = dict(ok, **kw)
        return f(a["c"], a["ldq"], a["rs"], a["M"], a["K"], a["w"], a["ldw"], a["s"], a["kind"], a["Gw"], a["N"],
                 a["b"], a["o"], a["ldo"], None)
    assert call(ldq=112) == ck.CK_ERR_INVALID_ARG        # ldq < K/2
    assert call(rs=None) == ck.CK_ERR_INVALID_ARG
    assert call(N=40) == ck.CK_ERR_UNSUPPORTED
    assert call(o=P + 64) == ck.CK_ERR_INVALID_ARG       # output overlaps the codes
    assert call(ldo=32) == ck.CK_ERR_INVALID_ARG
    assert call(M=0, c=None, rs=None, o=None) == ck.CK_OK


def test_quantize_weights_rejects():
    f = lib.ck_quantize_weights
    assert f(P, 4, 256, 256, 32, 0, P2, 128, P3, None) == ck.CK_ERR_UNSUPPORTED     # G
    assert f(P, 4, 320, 320, 256, 0, P2, 160, P3, None) == ck.CK_ERR_INVALID_ARG    # K % G
    assert f(P, 4, 256, 256, 64, 2, P2, 128, P3, None) == ck.CK_ERR_INVALID_ARG     # scale kind
    assert f(P, 4, 256, 200, 64, 0, P2, 128, P3, None) == ck.CK_ERR_INVALID_ARG     # ldw_in < K
    assert f(P + 8, 4, 256, 256, 64, 0, P2, 128, P3, None) == ck.CK_ERR_INVALID_ARG
    assert f(P, 4, 256, 256, 64, 0, P2, 120, P3, None) == ck.CK_ERR_INVALID_ARG     # ldp < K/2
    assert f(P, 4, 256, 256, 64, 0, P2, 136, P3, None) == ck.CK_ERR_INVALID_ARG     # ldp % 16
    assert f(P, 4, 256, 256, 64, 0, P2, 128, None, None) == ck.CK_ERR_INVALID_ARG
    assert f(P, 4, 256, 256, 64, 0, P + 64, 128, P3, None) == ck.CK_ERR_INVALID_ARG  # overlaps w
    assert f(P, 4, 256, 256, 64, 1, P2, 128, P2 + 256, None) == ck.CK_ERR_INVALID_ARG  # scales overlap packed
    assert f(P, -1, 256, 256, 64, 0, P2, 128, P3, None) == ck.CK_ERR_INVALID_ARG
    assert f(None, 0, 256, 256, 64, 0, None, 128, None, None) == ck.CK_OK


def test_test_hooks_reject():
    assert lib.ck_test_rotate_f32(P, 4, 256, 256, 64, P2 + 4, 256, None) == ck.CK_ERR_INVALID_ARG
    assert lib.ck_test_gemm_i32(P, 256, 4, 256, P3, 128, 64, P3, 64, None) == ck.CK_ERR_INVALID_ARG
    f = lib.ck_rotate_quant_packed4
    assert f(P, 4, 256, 256, 64, P2, 112, P3, None) == ck.CK_ERR_INVALID_ARG   # ldq < K/2
    assert f(P, 4, 256, 256, 64, P2, 136, P3, None) == ck.CK_ERR_INVALID_ARG   # ldq % 16
    assert f(P, 4, 256, 256, 64, P2 + 8, 128, P3, None) == ck.CK_ERR_INVALID_ARG
    assert f(P, 4, 256, 256, 64, P + 256, 128, P3, None) == ck.CK_ERR_INVALID_ARG  # overlaps x
    assert f(P, 4, 256, 256, 32, P2, 128, P3, None) == ck.CK_ERR_UNSUPPORTED
    assert f(None, 0, 256, 256, 64, None, 128, None, None) == ck.CK_OK
    g = lib.ck_test_gemm_i32_a4
    assert g(P, 112, 4, 256, P3, 128, 64, P4, 64, None) == ck.CK_ERR_INVALID_ARG    # ldq < K/2
    assert g(P, 128, 4, 256, P3, 128, 40, P4, 64, None) == ck.CK_ERR_UNSUPPORTED    # N % 16
    assert g(P, 128, 4, 256, P3, 128, 64, P3, 64, None) == ck.CK_ERR_INVALID_ARG    # acc overlaps
    assert g(P, 128, (1 << 22), 256, P3, 128, (1 << 22), P5, (1 << 22), None) == ck.CK_ERR_UNSUPPORTED


def test_noalloc_linear_rejects_before_any_hip_call():
    """The allocation-free linear validates like ck_w4a4_linear and refuses sizes beyond
    its 64 MiB + 64 KiB static scratch with CK_ERR_UNSUPPORTED, all before any HIP call."""
    f = lib.ck_w4a4_linear_noalloc

    def call(M=4, K=256, ldx=256, G=64, N=16, scale_kind=0, x_scale=1.0, out=P4, ldo=16):
        return f(P, M, K, ldx, G, P2, K // 2, P3, scale_kind, 64, N, None, x_scale, out, ldo, None)

    assert call(M=0) == ck.CK_OK
    assert call(G=32) == ck.CK_ERR_UNSUPPORTED
    assert call(K=96, ldx=96) == ck.CK_ERR_INVALID_ARG
    assert call(x_scale=0.0) == ck.CK_ERR_INVALID_ARG
    assert call(out=P + 64) == ck.CK_ERR_INVALID_ARG          # output overlaps x
    # packed codes of the tiled path: 8192 * 32768 / 2 = 128 MiB, beyond the scratch
    assert call(M=8192, K=32768, ldx=32768, N=16) == ck.CK_ERR_UNSUPPORTED
    assert b"static scratch" in lib.ck_last_error_msg()
    # 64 rows of 32768 fit, as do 8192 rows of 16384 (those would launch, so they are
    # not called here; tests/sanitize/abi_driver.cpp runs them against stub launchers)


def test_error_message_is_thread_local():
    import threading
    rq(G=32)
    msgs = []
    t = threading.Thread(target=lambda: msgs.append(lib.ck_last_error_msg()))
    t.start()
    t.join()
    assert msgs == [b""]
    assert b"G must be" in lib.ck_last_error_msg()


def test_binding_rejects_expanded_and_overlapping_rows():
    """Tensors whose rows overlap (an expanded row, a too-small row stride) are rejected
    by the binding before any call: the C ABI describes a matrix by one row stride and
    would read or write past the tensor's storage."""
    import torch
    M, K = 4, 256
    expanded = torch.zeros((1, K), dtype=torch.bfloat16).expand(M, K)
    assert expanded.stride(0) == 0
    with pytest.raises(ValueError, match="row stride"):
        ck.rotate_quant(expanded, 64, 8)
    overlapping = torch.zeros(M * K, dtype=torch.bfloat16).as_strided((M, K), (K // 2, 1))
    packed = torch.zeros((16, K // 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="row stride"):
        ck.linear(overlapping, 64, 8, packed, torch.zeros(16, dtype=torch.bfloat16), False)
    out = torch.zeros((1, 16), dtype=torch.bfloat16).expand(M, 16)
    with pytest.raises(ValueError, match="row stride"):
        ck._out(out, "out", torch.bfloat16, M, 16)
    with pytest.raises(ValueError, match="row stride"):
        ck._ld(expanded)
    # a single row may report any stride; dense and padded rows keep theirs
    assert ck._ld(torch.zeros((1, K)).as_strided((1, K), (0, 1))) == K
    assert ck._ld(torch.zeros((M, K + 64))[:, :K]) == K + 64


def test_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ck.rotate_quant(x, 64, 8)
