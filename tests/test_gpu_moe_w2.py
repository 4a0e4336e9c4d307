"""GPU parity of moe_lora_w2_delta (the routed down-projection delta, added to
y in place) against the fp64 oracle: weighted and unweighted, rows of
unadapted and invalid pairs left bitwise unchanged, the pair counts, both
arithmetic paths, ragged k and column tails, and the reduction to the dense
fused delta for one expert with top-1 (bitwise: the same partial order and
scale)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close, assert_close_chunked, assert_ws_ok, bf64, d16, d32, h16
from test_gpu_moe import check_pair_meta

pytestmark = pytest.mark.gpu

PATHS = {"default": 16, "valu": 1 << 30, "mfma": 1}


@pytest.fixture(params=list(PATHS))
def path(request):
    old = B.mfma_min_rows()
    B.set_mfma_min_rows(PATHS[request.param])
    yield request.param
    B.set_mfma_min_rows(old)


def device_tables(c: I.MoeW2Case):
    """Device banks and [E] pointer tables from fill_w_ptr: adapter l of expert
    e starts l * stride elements past entry e."""
    A, Bm = d16(c.a_down), d16(c.b_down)
    (ta, sa), (tb, sb) = B.fill_w_ptr(A), B.fill_w_ptr(Bm)
    assert (sa, sb) == (c.R * c.I, c.H * c.R)
    return (A, Bm), ta, sa, tb, sb


def run_w2(c: I.MoeW2Case, weighted: bool, ws=None, calls=None):
    """One call; returns (y rows as bf16 bits, counts, ws)."""
    keep, ta, sa, tb, sb = device_tables(c)
    y = d16(c.y)
    wt = d32(c.topk_weights) if weighted else None
    if ws is None:
        ws = B.moe_w2_workspace(c.T, c.top_k, c.E, c.L, c.R, c.I)
    B.moe_lora_w2_delta(d16(c.x2), ta, sa, tb, sb, d32(c.topk_ids), d32(c.lora_ids), c.R, y,
                        num_loras=c.L, topk_weights=wt, scale=c.scale, ws=ws)
    assert_ws_ok(ws, moe=True, calls=calls)
    del keep
    return h16(y), B.moe_counts(ws).cpu().numpy(), ws


def check_w2(c: I.MoeW2Case, weighted: bool, what="", ws=None, calls=None):
    """Every routed pair against the oracle, unrouted rows bitwise, counts
    and pair metadata bit-exact."""
    print(f"moe w2 case T={c.T} E={c.E} L={c.L} I={c.I} H={c.H} R={c.R} weighted={weighted} {what}",
          flush=True)
    out, counts, ws = run_w2(c, weighted, ws, calls)
    lora = np.repeat(c.lora_ids, c.top_k)
    ex = c.topk_ids.reshape(-1)
    valid = (lora >= 0) & (lora < c.L) & (ex >= 0) & (ex < c.E)
    assert np.array_equal(out[~valid], c.y[~valid]), "unrouted pairs must keep y bit for bit"
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    _, _, _, ocnt = O.meta_build(keys, c.E * c.L)
    assert counts.tolist() == ocnt.tolist()
    check_pair_meta(c, ws)
    return assert_close_chunked(out, lambda p: O.case_moe_w2_pairs(c, p, weighted), np.flatnonzero(valid),
                                f"moe w2 weighted={weighted} {what}", chunk=2048)


def small_w2(seed, **kw):
    args = dict(T=50, H=264, E=5, top_k=3, I=40, R=16, L=3, neg_frac=0.2, scale=0.75)
    args.update(kw)
    c = I.make_moe_w2(seed, **args)
    rng = np.random.default_rng(seed + 100)
    c.lora_ids[rng.random(c.T) < 0.05] = c.L + 1               # invalid adapter ids
    c.topk_ids[rng.random(c.topk_ids.shape) < 0.03] = c.E + 2  # invalid expert ids
    return c


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("seed", [1, 2])
def test_w2_small(seed, weighted, path):
    # seed 2: three experts, so (adapter, expert) segments run past 16 rows
    c = small_w2(seed, T=60 if seed == 1 else 400, E=5 if seed == 1 else 3)
    check_w2(c, weighted, what=f"seed={seed} {path}")


@pytest.mark.parametrize("R", [8, 32, 64, 128])
def test_w2_ragged_k_and_columns(R, path):
    # I = 1032: three k pieces, the last 8 wide; H = 1096: column tail of 72
    c = small_w2(3, T=90, E=2, top_k=2, I=1032, H=1096, R=R, L=2)
    check_w2(c, True, what=f"R={R} {path}")


def test_w2_wide_columns(path):
    # 8000 pairs over 16 keys: about 516 tiles, so the expand units widen to
    # 1024 columns (two 512-column batches, the last unit ragged)
    c = small_w2(4, T=4000, E=4, top_k=2, I=264, H=2056, R=16, L=4, neg_frac=0.05)
    check_w2(c, True, what=f"wide {path}")


def test_w2_no_pairs():
    c = small_w2(5, T=0)
    out, counts, _ = run_w2(c, True)
    assert out.size == 0 and counts.tolist() == [0, 0, 0, 0]


def test_w2_single_expert_top1_matches_dense_fused():
    c = small_w2(6, T=130, E=1, top_k=1, L=4, I=520, H=520, R=16, neg_frac=0.2)
    c.lora_ids[c.lora_ids >= c.L] = -1
    c.topk_ids[:] = 0
    out, _, _ = run_w2(c, False)
    a_pool = d16(np.ascontiguousarray(c.a_down[0][:, None]))   # [L, 1, R, I]
    b_pool = d16(np.ascontiguousarray(c.b_down[0]))            # [L, H, R]
    y = d16(c.y)
    meta = B.lora_meta_build(d32(c.lora_ids), c.L)
    ws = B.fused_workspace(c.T, c.L, 1, c.R, c.I)
    B.lora_delta_fused(d16(c.x2), a_pool, b_pool, torch.full((c.L,), c.scale, device="cuda"), (c.H,),
                       meta, y, ws=ws)
    assert_ws_ok(ws, calls=1)
    # one expert at top-1 is the dense delta with the adapter as slot: the two
    # calls (different kernels, different summation order) agree within the
    # tolerance, and both match the oracle
    dense = h16(y)
    rows = np.flatnonzero((c.lora_ids >= 0) & (c.lora_ids < c.L))
    assert np.array_equal(out[c.lora_ids < 0], c.y[c.lora_ids < 0])
    assert np.array_equal(dense[c.lora_ids < 0], c.y[c.lora_ids < 0])
    orc = O.case_moe_w2_pairs(c, rows, False)
    assert_close(bf64(out[rows]), orc, "w2 at E=1, top-1")
    assert_close(bf64(dense[rows]), orc, "dense fused at E=1, top-1")
    assert_close(bf64(out[rows]), bf64(dense[rows]), "w2 vs dense fused")


def test_w2_unit_weights_equal_unweighted():
    c = small_w2(7, T=200, E=3)
    c.topk_weights[:] = 1.0
    a, _, _ = run_w2(c, True)
    b, _, _ = run_w2(c, False)
    assert np.array_equal(a, b)


@pytest.fixture(scope="module")
def w2_case():
    return I.moe_w2()


def test_w2_config_full(w2_case):
    check_w2(w2_case, True, what="config")


def test_w2_deterministic(w2_case):
    c = w2_case
    ws = B.moe_w2_workspace(c.T, c.top_k, c.E, c.L, c.R, c.I)
    a, _, _ = run_w2(c, True, ws, calls=1)
    b, _, _ = run_w2(c, True, ws, calls=2)
    assert np.array_equal(a, b)


def test_w2_config_reusing_its_routing(w2_case):
    """The full w2 config as the bench times it with reused routing: a call
    that builds the pair metadata, then one that reuses it on a fresh y, bit
    for bit the same (the first is checked against the oracle in full by
    test_w2_config_full); the metadata left in the workspace is the oracle's."""
    c = w2_case
    ws = B.moe_w2_workspace(c.T, c.top_k, c.E, c.L, c.R, c.I)
    first, _, _ = run_w2(c, True, ws, calls=1)
    keep, ta, sa, tb, sb = device_tables(c)
    y = d16(c.y)
    B.moe_lora_w2_delta(d16(c.x2), ta, sa, tb, sb, d32(c.topk_ids), d32(c.lora_ids), c.R, y,
                        num_loras=c.L, topk_weights=d32(c.topk_weights), scale=c.scale, ws=ws,
                        reuse_routing=True)
    assert_ws_ok(ws, moe=True, calls=2)
    assert np.array_equal(h16(y), first)
    check_pair_meta(c, ws)
    del keep


def test_w2_workspace_reused_across_shapes(w2_case):
    """One workspace, calls of different T in turn, each with its own inputs
    and routing (big, small, big, big): each matches the oracle on every
    routed pair, and the control line counts every call with no error."""
    c = w2_case
    small = small_w2(8, T=70, E=c.E, top_k=c.top_k, L=c.L, I=c.I, R=c.R, H=c.H)
    big2 = I.make_moe_w2(34, T=c.T, H=c.H, E=c.E, top_k=c.top_k, I=c.I, R=c.R, L=c.L)
    big3 = I.make_moe_w2(35, T=c.T, H=c.H, E=c.E, top_k=c.top_k, I=c.I, R=c.R, L=c.L)
    ws = B.moe_w2_workspace(c.T, c.top_k, c.E, c.L, c.R, c.I)
    for i, case in enumerate([c, small, big2, big3]):
        check_w2(case, True, what=f"reuse call {i}", ws=ws, calls=i + 1)


def test_w2_reuses_the_gemm1_routing():
    """The down projection after gemm1 on one workspace: with reuse_routing the
    pair metadata gemm1 built is used as is, and the result is bit for bit the
    one of a call that builds it."""
    c = small_w2(9, T=300, E=4, top_k=2, I=264, H=520, R=16, L=3)
    g = I.make_moe(9, T=c.T, H=136, E=c.E, top_k=c.top_k, I=64, R=c.R, L=c.L)
    g.topk_ids[:] = c.topk_ids
    g.lora_ids[:] = c.lora_ids
    n1 = int(B.lib().moe_lora_workspace_bytes(c.T, c.top_k, c.E, c.L, c.R, g.H))
    n2 = int(B.lib().moe_lora_w2_workspace_bytes(c.T, c.top_k, c.E, c.L, c.R, c.I))
    ws = torch.zeros(max(n1, n2), dtype=torch.uint8, device="cuda")
    # gemm1 on the shared workspace builds the routing
    Ag, Au, Bg, Bu = d16(g.a_gate), d16(g.a_up), d16(g.b_gate), d16(g.b_up)
    (ta, sa1), (tb, sb1) = B.fill_w_ptr(Ag, Au), B.fill_w_ptr(Bg, Bu)
    B.moe_lora_gemm1_delta(d16(g.x), ta, sa1, tb, sb1, d32(g.topk_ids), d32(g.lora_ids), g.R,
                           g.I, num_loras=g.L, ws=ws)
    assert_ws_ok(ws, moe=True, calls=1)
    keep, wa, sa, wb, sb = device_tables(c)
    y_reuse = d16(c.y)
    B.moe_lora_w2_delta(d16(c.x2), wa, sa, wb, sb, d32(c.topk_ids), d32(c.lora_ids), c.R, y_reuse,
                        num_loras=c.L, topk_weights=d32(c.topk_weights), scale=c.scale, ws=ws,
                        reuse_routing=True)
    assert_ws_ok(ws, moe=True, calls=2)
    fresh, _, _ = run_w2(c, True)
    assert np.array_equal(h16(y_reuse), fresh)
    del keep
