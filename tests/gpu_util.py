"""Helpers shared by the GPU parity tests (host <-> device marshalling only)."""
import numpy as np
import torch

import workloads

DEV = torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def i8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def assert_codes_close(gpu: np.ndarray, ref: np.ndarray, min_equal: float = 0.9999):
    """Rotation codes: at least `min_equal` of the elements identical, none off by more than 1."""
    d = np.abs(gpu.astype(np.int32) - ref.astype(np.int32))
    assert d.max() <= 1, "a code differs by %d" % d.max()
    frac = float((d == 0).mean())
    assert frac >= min_equal, "only %.6f of the codes agree" % frac


def assert_output_close(gpu: np.ndarray, ref: np.ndarray):
    """bf16 outputs: max |err| <= 1e-2 (|ref| + 1), and within bf16 rounding plus fp32 noise."""
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = 1e-2 * (np.abs(ref) + 1.0)
    assert (err <= bound).all(), "max err %.3g (bound violated at %d places)" % (err.max(), (err > bound).sum())
    tight = 2.0 ** -8 * np.abs(ref) + 1e-4 * (np.abs(ref).max() + 1.0)
    assert (err <= tight).all(), "error above bf16 rounding: max %.3g" % (err - tight).max()
