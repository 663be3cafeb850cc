"""Seeded synthetic inputs for the ConvRot packed-INT4 linear.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no rotation, quantisation, packing or matmul), so
that the oracle and the GPU path can share it.  Every array is produced on the
host from numpy's PCG64 generator; bf16 data is returned as uint16 bit
patterns (fp64 draw -> fp32 -> bf16, round to nearest even via torch's CPU
conversion).

Recipe (stated once, used everywhere):
  * activations: N(0,1) draws; a set of outlier columns, drawn without
    replacement and shared by all rows, is multiplied by 20; listed rows are
    set to zero; when the row stride exceeds K the padding columns hold a bf16
    NaN so that an out-of-row read shows up in the results;
  * packed weights: independent uniform bytes, which is the same as two
    independent uniform 4-bit codes per byte;
  * weight scales: uniform in [0.002, 0.02], rounded to bf16;
  * AWQ zero points: N(0, 0.01^2) (sigma 0.01), rounded to bf16.
Each array of a workload comes from its own child stream of
SeedSequence(seed), so changing one shape does not move the others.
"""
from __future__ import annotations

import numpy as np

BF16_NAN = 0x7FC0

# Workloads, named by what they are.  "scale" is the weight-scale kind:
# "group" = bf16 [K/64, N], "channel" = bf16 [N].
WORKLOADS = {
    "w4a8_linear_m32_k3840_n3840_g64": dict(
        M=32, K=3840, N=3840, G=64, bits=8, scale="group", Gw=64, seed=0, outliers=8),
    "w4a8_decode_gemv_k3840_n10240_g64": dict(
        Ms=(1, 4, 8), K=3840, N=10240, G=64, bits=8, scale="group", Gw=64, seed=1, outliers=8),
    "w4a4_linear_m8192_k3840_n3840_g64": dict(
        M=8192, K=3840, N=3840, G=64, bits=4, scale="channel", Gw=64, seed=2, outliers=38),
    "w4a4_linear_m8192_k10240_n3840_g256": dict(
        M=8192, K=10240, N=3840, G=256, bits=4, scale="channel", Gw=64, seed=3, outliers=102,
        zero_rows=(0, 127, 128, 4095, 8191)),
    "rotate_quant_m8192_k10240_ld10752": dict(
        M=8192, K=10240, ld=10752, Gs=(16, 64, 256), bits=8, seed=4, outliers=102),
    "awq_w4a16_gemv_m1_k3072_n18432": dict(M=1, K=3072, N=18432, Gw=64, seed=4),
}

# child-stream numbers inside one workload's SeedSequence
_S_X, _S_W, _S_SCALE, _S_ZERO, _S_BIAS, _S_AWQ_X = range(6)


def _rng(seed: int, stream: int) -> np.random.Generator:
    child = np.random.SeedSequence(seed).spawn(stream + 1)[stream]
    return np.random.Generator(np.random.PCG64(child))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64/fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(M: int, K: int, seed: int, outliers: int = 0, ld: int | None = None,
                zero_rows=(), stream: int = _S_X) -> np.ndarray:
    """bf16 bits [M, ld]: N(0,1) with `outliers` columns x20 and the given zero rows."""
    ld = K if ld is None else ld
    rng = _rng(seed, stream)
    x = rng.standard_normal((M, K))
    if outliers:
        cols = rng.choice(K, size=outliers, replace=False)
        x[:, cols] *= 20.0
    for r in zero_rows:
        if r < M:
            x[r, :] = 0.0
    out = np.full((M, ld), BF16_NAN, dtype=np.uint16)
    out[:, :K] = to_bf16_bits(x)
    return out


def packed_weights(N: int, K: int, seed: int, ld: int | None = None) -> np.ndarray:
    """uint8 [N, ld] with K/2 uniform random bytes per row (padding bytes 0xA5)."""
    ld = K // 2 if ld is None else ld
    rng = _rng(seed, _S_W)
    out = np.full((N, ld), 0xA5, dtype=np.uint8)
    out[:, :K // 2] = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    return out


def uniform_bf16(shape, lo: float, hi: float, seed: int, stream: int = _S_SCALE) -> np.ndarray:
    return to_bf16_bits(_rng(seed, stream).uniform(lo, hi, size=shape))


def normal_bf16(shape, sigma: float, seed: int, stream: int = _S_ZERO) -> np.ndarray:
    return to_bf16_bits(_rng(seed, stream).normal(0.0, sigma, size=shape))


def weight_scales(kind: str, K: int, N: int, seed: int, Gw: int = 64) -> np.ndarray:
    shape = (K // Gw, N) if kind == "group" else (N,)
    return uniform_bf16(shape, 0.002, 0.02, seed)


def bias(N: int, seed: int) -> np.ndarray:
    return normal_bf16((N,), 0.5, seed, stream=_S_BIAS)


def linear_inputs(M: int, K: int, N: int, seed: int, outliers: int, scale: str, Gw: int = 64,
                  zero_rows=(), ld: int | None = None, with_bias: bool = False) -> dict:
    """Everything one ConvRot linear call needs, as host arrays."""
    d = dict(
        x=activations(M, K, seed, outliers, ld=ld, zero_rows=zero_rows),
        packed=packed_weights(N, K, seed),
        w_scales=weight_scales(scale, K, N, seed, Gw),
        per_group=(scale == "group"),
        Gw=Gw,
        K=K,
    )
    d["bias"] = bias(N, seed) if with_bias else None
    return d


def awq_inputs(M: int, K: int, N: int, seed: int, Gw: int = 64, with_bias: bool = False) -> dict:
    return dict(
        x=activations(M, K, seed, 0, stream=_S_AWQ_X),
        packed=packed_weights(N, K, seed),
        scales=uniform_bf16((K // Gw, N), 0.002, 0.02, seed),
        zeros=normal_bf16((K // Gw, N), 0.01, seed),
        Gw=Gw,
        K=K,
        bias=bias(N, seed) if with_bias else None,
    )


def workload_inputs(name: str, M: int | None = None) -> dict:
    """Inputs of a named workload (M overrides the row count, e.g. for decode)."""
    w = WORKLOADS[name]
    if name.startswith("awq"):
        return awq_inputs(M or w["M"], w["K"], w["N"], w["seed"], w["Gw"])
    if name.startswith("rotate_quant"):
        return dict(x=activations(M or w["M"], w["K"], w["seed"], w["outliers"], ld=w["ld"]),
                    K=w["K"])
    m = M or w.get("M") or w["Ms"][0]
    return linear_inputs(m, w["K"], w["N"], w["seed"], w["outliers"], w["scale"], w["Gw"],
                         zero_rows=w.get("zero_rows", ()))
