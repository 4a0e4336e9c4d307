"""GPU parity of moe_lora_gemm1_delta (regular and shared-A forms) against the
fp64 oracle: per-(token, slot) gate/up deltas on every pair, zero rows for
unadapted and invalid pairs (bitwise), the pair metadata the call builds in
its workspace (bit for bit), the workspace control line after every call,
and shared-A == regular when the adapters share A."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close, assert_close_chunked, assert_ws_ok, bf64, d16, d32, h16
from test_gpu_meta import assert_meta_matches

pytestmark = pytest.mark.gpu

PATHS = {"default": 16, "valu": 1 << 30, "mfma": 1}


@pytest.fixture(params=list(PATHS))
def path(request):
    old = B.mfma_min_rows()
    B.set_mfma_min_rows(PATHS[request.param])
    yield request.param
    B.set_mfma_min_rows(old)


def device_tables(c: I.MoeCase, shared: bool):
    """Device banks and FlashInfer-style pointer tables ([2, E] or [E]) from fill_w_ptr."""
    if shared:
        A, Bm = d16(c.a_shared), d16(c.b_fused)
        (ta, sa), (tb, sb) = B.fill_w_ptr(A), B.fill_w_ptr(Bm)
        assert (sa, sb) == (c.R * c.H, 2 * c.I * c.R)
        return (A, Bm), ta, sa, tb, sb
    Ag, Au, Bg, Bu = d16(c.a_gate), d16(c.a_up), d16(c.b_gate), d16(c.b_up)
    (ta, sa), (tb, sb) = B.fill_w_ptr(Ag, Au), B.fill_w_ptr(Bg, Bu)
    assert ta.shape == (2, c.E) and (sa, sb) == (c.R * c.H, c.I * c.R)
    return (Ag, Au, Bg, Bu), ta, sa, tb, sb


SENTINEL = 0x40E0   # bf16 bits of 7.0, the fill of `out` before the call


def run_moe(c: I.MoeCase, shared: bool, ws=None, calls=None):
    """One call; returns (out rows [T*top_k, 2I] as bf16 bits, counts, ws)."""
    keep, ta, sa, tb, sb = device_tables(c, shared)
    x = d16(c.x)
    if ws is None:
        ws = B.moe_workspace(c.T, c.top_k, c.E, c.L, c.R, c.H)
    out = torch.full((c.T, c.top_k, 2 * c.I), 7.0, dtype=torch.bfloat16, device="cuda")
    B.moe_lora_gemm1_delta(x, ta, sa, tb, sb, d32(c.topk_ids), d32(c.lora_ids), c.R, c.I,
                           num_loras=c.L, scale=c.scale, out=out, ws=ws)
    assert_ws_ok(ws, moe=True, calls=calls)
    del keep
    return h16(out).reshape(c.T * c.top_k, 2 * c.I), B.moe_counts(ws).cpu().numpy(), ws


def check_pair_meta(c, ws):
    """The pair metadata the call built in its workspace equals the oracle's
    metadata of the (adapter, expert) keys, bit for bit."""
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    assert_meta_matches(B.moe_meta_view(ws, c.T, c.top_k, c.E, c.L), keys, c.E * c.L)


def check_moe(c: I.MoeCase, shared: bool, what="", ws=None, calls=None):
    """Every pair against the oracle, zero rows bitwise, counts and pair
    metadata bit-exact, no pair left holding the pre-call fill."""
    print(f"moe case T={c.T} E={c.E} L={c.L} shared={shared} {what}", flush=True)
    out, counts, ws = run_moe(c, shared, ws, calls)
    n = c.T * c.top_k
    lora = np.repeat(c.lora_ids, c.top_k)
    ex = c.topk_ids.reshape(-1)
    valid = (lora >= 0) & (lora < c.L) & (ex >= 0) & (ex < c.E)
    assert not out[~valid].any(), "pairs without a valid (adapter, expert) must be zero rows"
    assert not (out[valid] == SENTINEL).all(axis=1).any(), "a routed pair's row was never written"
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    _, _, _, ocnt = O.meta_build(keys, c.E * c.L)
    assert counts.tolist() == ocnt.tolist()
    check_pair_meta(c, ws)
    return assert_close_chunked(out, lambda p: O.case_moe_pairs(c, shared, p), np.arange(n),
                                f"moe shared={shared} {what}", chunk=2048)


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
    o_reg, _, _ = run_moe(c, False)
    o_sh, _, _ = run_moe(c, True)
    assert_close(bf64(o_reg), bf64(o_sh), "shared vs regular")


@pytest.fixture(scope="module")
def moe_case():
    return I.moe_gemm1()


@pytest.mark.parametrize("shared", [False, True])
def test_moe_config_full(moe_case, shared):
    check_moe(moe_case, shared, what="config")


def test_moe_deterministic(moe_case):
    ws = B.moe_workspace(moe_case.T, moe_case.top_k, moe_case.E, moe_case.L, moe_case.R, moe_case.H)
    a, _, _ = run_moe(moe_case, False, ws, calls=1)
    b, _, _ = run_moe(moe_case, False, ws, calls=2)
    assert np.array_equal(a, b)


def test_moe_no_pairs():
    c = small_moe(9, T=0)
    out, counts, _ = run_moe(c, False)
    assert out.size == 0 and counts.tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("seed", [21, 22])
def test_moe_pair_metadata_small_split(seed):
    """At most 1024 pairs: (adapter, expert) segments of 9..15 pairs are cut
    into two tiles; invalid adapter and expert ids are counted."""
    c = small_moe(seed, T=60, E=5, top_k=3, L=3)
    assert c.T * c.top_k <= 1024
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    lens = np.bincount(keys[(keys >= 0) & (keys < c.E * c.L)], minlength=c.E * c.L)
    assert ((lens > 8) & (lens < 16)).any(), "the case must hold a segment that is cut in two"
    check_moe(c, False, what=f"split seed={seed}")


def test_moe_workspace_reused_across_shapes(moe_case):
    """One workspace, calls of different T in turn, each with its own tokens
    and routing: big, small, big, big.  The control line stays at one place
    whatever the shape, so every call gets a fresh tag and no call takes an
    earlier call's partials; each call matches the oracle on every pair."""
    c = moe_case
    small = I.make_moe(31, T=70, H=c.H, E=c.E, top_k=c.top_k, I=c.I, R=c.R, L=c.L)
    big2 = I.make_moe(32, T=c.T, H=c.H, E=c.E, top_k=c.top_k, I=c.I, R=c.R, L=c.L)
    big3 = I.make_moe(33, T=c.T, H=c.H, E=c.E, top_k=c.top_k, I=c.I, R=c.R, L=c.L)
    ws = B.moe_workspace(c.T, c.top_k, c.E, c.L, c.R, c.H)
    for i, case in enumerate([c, small, big2, big3]):
        check_moe(case, False, what=f"reuse call {i}", ws=ws, calls=i + 1)


def test_moe_meta_counters_survive_shapes():
    """One workspace, pair metadata built two ways in turn: 32768 pairs over
    512 (adapter, expert) keys (too many chunks for the per-chunk slot table:
    one workgroup assembles, taking a ticket) and 16384 pairs (one assembling
    workgroup per chunk).  Each shape's metadata regions cover the other's
    metadata workspace, so the build's counters (the ticket and the invalid
    pair count) must sit where no shape writes anything else; every call is
    compared in full, its counts and pair metadata bit for bit."""
    kw = dict(H=264, E=64, top_k=8, I=40, R=16, L=8, neg_frac=0.1)
    cases = []
    for i, T in enumerate([4096, 2048, 4096, 2048]):
        c = I.make_moe(51 + i, T=T, **kw)
        rng = np.random.default_rng(51 + i)
        c.lora_ids[rng.random(c.T) < 0.02] = c.L + 1
        c.topk_ids[rng.random(c.topk_ids.shape) < 0.01] = c.E + 2
        cases.append(c)
    ws = B.moe_workspace(4096, 8, 64, 8, 16, 264)
    for i, c in enumerate(cases):
        check_moe(c, False, what=f"counters call {i} T={c.T}", ws=ws, calls=i + 1)


@pytest.mark.parametrize("shared", [False, True])
def test_moe_segments_longer_than_64_pairs(shared):
    """A hot expert: its (adapter, expert) segments run past 64 pairs (their
    later groups of 64 are taken by further units) while the call averages
    well under 64 pairs per key, the regime of one workgroup per segment."""
    c = small_moe(23, T=300, E=8, top_k=2, L=2, H=520, I=72)
    c.topk_ids[:200, 0] = 0                      # 200 tokens route to expert 0 first
    c.topk_ids[:200, 1] = np.where(c.topk_ids[:200, 1] == 0, 1, c.topk_ids[:200, 1])
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    lens = np.bincount(keys[(keys >= 0) & (keys < c.E * c.L)], minlength=c.E * c.L)
    assert lens.max() > 64 and (keys >= 0).sum() <= 64 * c.E * c.L
    check_moe(c, shared, what="long segments")


@pytest.mark.parametrize("R", [32, 128])
@pytest.mark.parametrize("shared", [False, True])
def test_moe_ranks_32_and_128(R, shared, path):
    """Rank 32 on the segment kernel (four rank groups in the regular form,
    two in the shared one) and rank 128, the largest rank taken, on the fused
    kernel (256 rank rows in the regular form)."""
    c = small_moe(43, T=200, H=264, E=3, top_k=2, I=72, R=R, L=2)
    check_moe(c, shared, f"R={R} {path}")


@pytest.mark.parametrize("shared", [False, True])
def test_moe_small_rank_many_pairs_per_key(shared, path):
    """More than 64 pairs per (adapter, expert) key on average: rank 16 takes
    the fused kernel, which spreads a long segment over many workgroups."""
    c = small_moe(44, T=300, H=264, E=2, top_k=1, I=40, R=16, L=1, neg_frac=0.1)
    assert c.T * c.top_k > 64 * c.E * c.L
    check_moe(c, shared, f"many pairs per key {path}")


@pytest.mark.parametrize("shared", [False, True])
def test_moe_rank64_wide_fused(shared, path):
    """Rank 64 takes the fused kernel (the segment kernel serves ranks 8, 16
    and 32); with long segments and 8200-column windows its units are wide:
    on the MFMA path the shrink pairs tiles (128 rank rows in the regular
    form) and the expand stages B through LDS from whole-row loads."""
    c = small_moe(41, T=512, H=264, E=2, top_k=2, I=8200, R=64, L=1, neg_frac=0.1)
    check_moe(c, shared, f"rank 64 wide {path}")
