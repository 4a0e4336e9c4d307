"""Helpers shared by the GPU parity tests: host <-> device copies of bf16 bit
patterns, the element-wise tolerance check |gpu - oracle| <= 1e-2 + 2e-2 |oracle|,
chunked full-size comparison against the oracle, and the workspace control
line check (no bounded wait gave up, no call left half counted)."""
import numpy as np
import torch

from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B

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


def assert_close_chunked(gpu_bits: np.ndarray, oracle_of, idx: np.ndarray, what: str, chunk: int = 256):
    """Compare gpu_bits[idx] (bf16 rows) with oracle_of(idx_chunk) chunk by
    chunk, so that no full-size fp64 array is ever held; every index is
    compared.  Returns the worst err/tol."""
    idx = np.asarray(idx)
    worst = 0.0
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        worst = max(worst, assert_close(bf64(gpu_bits[sel]), oracle_of(sel), f"{what} [{c0}:{c0 + sel.size}]"))
    return worst


def assert_ws_ok(ws: torch.Tensor, moe: bool = False, calls: int | None = None):
    """The workspace's control line after the stream reached the last call:
    error word 0, no tiles left counted, and (when given) the number of calls
    completed on it; the metadata build's two counters, at byte 64 of a fused
    or MoE workspace, back to zero."""
    torch.cuda.synchronize()
    st = B.ws_status(ws, moe)
    assert st.error == 0, f"a bounded wait gave up: {st}"
    assert st.running == 0, f"a call left tiles counted: {st}"
    assert ws[64:72].view(torch.int32).cpu().tolist() == [0, 0], "the metadata build left a counter set"
    if calls is not None:
        assert st.calls == calls, st
    return st
