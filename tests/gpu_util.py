"""Helpers shared by the GPU parity tests: host <-> device copies of bf16 bit
patterns and the element-wise tolerance check |gpu - oracle| <= 1e-2 + 2e-2 |oracle|."""
import numpy as np
import torch

from tenant_lora_serving_amd import inputs as I

ATOL, RTOL = 1e-2, 2e-2


def d16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def h16(t: torch.Tensor) -> np.ndarray:
    """device bfloat16 -> host uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def d32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def assert_close(gpu: np.ndarray, orc: np.ndarray, what: str):
    gpu = np.asarray(gpu, dtype=np.float64)
    orc = np.asarray(orc, dtype=np.float64)
    assert gpu.shape == orc.shape, (gpu.shape, orc.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - orc)
    tol = ATOL + RTOL * np.abs(orc)
    bad = err > tol
    worst = float((err / tol).max()) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside "
                           f"1e-2 + 2e-2|o| (worst err/tol {worst:.3f})")
    return worst
