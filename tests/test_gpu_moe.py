"""GPU parity of moe_lora_gemm1_delta (regular and shared-A forms) against the
fp64 oracle: per-(token, slot) gate/up deltas, zero rows for unadapted and
invalid pairs (bitwise), the pair counts, and shared-A == regular when the
adapters share A."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close, bf64, d16, d32, h16

pytestmark = pytest.mark.gpu

PATHS = {"default": 16, "valu": 1 << 30, "mfma": 1}


@pytest.fixture(params=list(PATHS))
def path(request):
    old = B.mfma_min_rows()
    B.set_mfma_min_rows(PATHS[request.param])
    yield request.param
    B.set_mfma_min_rows(old)


def device_tables(c: I.MoeCase, shared: bool):
    """Device banks and FlashInfer-style pointer tables ([2, E] or [E])."""
    E, L, R, H, I_ = c.E, c.L, c.R, c.H, c.I
    if shared:
        A, Bm = d16(c.a_shared), d16(c.b_fused)
        ta = torch.tensor([A.data_ptr() + e * L * R * H * 2 for e in range(E)], dtype=torch.int64)
        tb = torch.tensor([Bm.data_ptr() + e * L * 2 * I_ * R * 2 for e in range(E)], dtype=torch.int64)
        return (A, Bm), ta.cuda(), R * H, tb.cuda(), 2 * I_ * R
    Ag, Au, Bg, Bu = d16(c.a_gate), d16(c.a_up), d16(c.b_gate), d16(c.b_up)
    ta = torch.tensor([[M.data_ptr() + e * L * R * H * 2 for e in range(E)] for M in (Ag, Au)],
                      dtype=torch.int64)
    tb = torch.tensor([[M.data_ptr() + e * L * I_ * R * 2 for e in range(E)] for M in (Bg, Bu)],
                      dtype=torch.int64)
    return (Ag, Au, Bg, Bu), ta.cuda(), R * H, tb.cuda(), I_ * R


def run_moe(c: I.MoeCase, shared: bool, ws=None):
    keep, ta, sa, tb, sb = device_tables(c, shared)
    x = d16(c.x)
    if ws is None:
        ws = B.moe_workspace(c.T, c.top_k, c.E, c.L, c.R, c.H)
    out = torch.full((c.T, c.top_k, 2 * c.I), 7.0, dtype=torch.bfloat16, device="cuda")
    B.moe_lora_gemm1_delta(x, ta, sa, tb, sb, d32(c.topk_ids), d32(c.lora_ids), c.R, c.I,
                           num_loras=c.L, scale=c.scale, out=out, ws=ws)
    torch.cuda.synchronize()
    del keep
    return h16(out).reshape(c.T * c.top_k, 2 * c.I), B.moe_counts(ws).cpu().numpy()


def check_moe(c: I.MoeCase, shared: bool, sample=None, what=""):
    print(f"moe case T={c.T} E={c.E} L={c.L} shared={shared} {what}", flush=True)
    out, counts = run_moe(c, shared)
    n = c.T * c.top_k
    lora = np.repeat(c.lora_ids, c.top_k)
    ex = c.topk_ids.reshape(-1)
    valid = (lora >= 0) & (lora < c.L) & (ex >= 0) & (ex < c.E)
    assert not out[~valid].any(), "pairs without a valid (adapter, expert) must be zero rows"
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    _, _, _, ocnt = O.meta_build(keys, c.E * c.L)
    assert counts.tolist() == ocnt.tolist()
    pairs = np.arange(n) if sample is None else np.unique(np.concatenate([
        np.flatnonzero(valid)[:: max(1, valid.sum() // sample)], np.flatnonzero(~valid)[:8]]))
    orc = O.case_moe_pairs(c, shared, pairs)
    return assert_close(bf64(out[pairs]), orc, f"moe shared={shared} {what}")


def small_moe(seed, **kw):
    args = dict(T=50, H=264, E=5, top_k=3, I=40, R=16, L=3, neg_frac=0.2, scale=0.75)
    args.update(kw)
    c = I.make_moe(seed, **args)
    rng = np.random.default_rng(seed)
    bad = rng.random(c.T) < 0.05
    c.lora_ids[bad] = c.L + 1                       # invalid adapter ids
    badp = rng.random(c.topk_ids.shape) < 0.03
    c.topk_ids[badp] = c.E + 2                      # invalid expert ids
    return c


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("seed", [1, 2])
def test_moe_small(seed, shared, path):
    c = small_moe(seed, T=60 if seed == 1 else 400, E=5 if seed == 1 else 3)
    check_moe(c, shared, what=f"seed={seed} {path}")


def test_moe_single_expert_top1(path):
    c = small_moe(3, T=77, E=1, top_k=1, L=4, I=24, R=8)
    check_moe(c, False, what=path)
    check_moe(c, True, what=path)


def test_moe_shared_equals_regular_when_a_shared():
    c = small_moe(4, T=120)
    c.a_gate[:] = c.a_shared
    c.a_up[:] = c.a_shared
    c.b_gate[:] = c.b_fused[:, :, :c.I]
    c.b_up[:] = c.b_fused[:, :, c.I:]
    o_reg, _ = run_moe(c, False)
    o_sh, _ = run_moe(c, True)
    assert_close(bf64(o_reg), bf64(o_sh), "shared vs regular")


@pytest.fixture(scope="module")
def moe_case():
    return I.moe_gemm1()


@pytest.mark.parametrize("shared", [False, True])
def test_moe_config_full(moe_case, shared):
    check_moe(moe_case, shared, sample=400, what="config")


def test_moe_deterministic(moe_case):
    ws = B.moe_workspace(moe_case.T, moe_case.top_k, moe_case.E, moe_case.L, moe_case.R, moe_case.H)
    a, _ = run_moe(moe_case, False, ws)
    b, _ = run_moe(moe_case, False, ws)
    assert np.array_equal(a, b)


def test_moe_no_pairs():
    c = small_moe(9, T=0)
    out, counts = run_moe(c, False)
    assert out.size == 0 and counts.tolist() == [0, 0, 0, 0]
