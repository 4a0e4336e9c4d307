"""GPU parity at the largest shapes the boundary accepts: n = 2^22 rows (or
(token, slot) pairs) over 8192 slots, the most a build that spans several
1024-row chunks takes.  Metadata is compared bit for bit in full; the delta
on a sample of rows (the first and last rows, the rows of the first and last
segments, and random ones), and every row that gets no delta is compared
bitwise in full.  Widths and rank are small, so the oracle stays cheap while
every index that grows with n (rows, tiles, pieces, chunks) reaches its
largest value.  MoE gemm1 and w2 take 2^19 tokens x top_k 8 over 64 experts
x 128 adapters."""
import numpy as np
import pytest

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from gpu_util import assert_close_chunked, h16
from test_gpu_dense import Dev, active, check_y, small_case
from test_gpu_meta import check_meta
from test_gpu_moe import SENTINEL, check_pair_meta, run_moe
from test_gpu_moe_w2 import run_w2

pytestmark = pytest.mark.gpu

N_MAX = 1 << 22
S_MULTI_MAX = 8192


def sample_rows(rng, keys, S, k=3000):
    """First and last rows, the rows of the first and last segments (the
    smallest and largest active key, in row order), random rows."""
    n = keys.size
    act = (keys >= 0) & (keys < S)
    first = np.flatnonzero(keys == keys[act].min())[:64]
    last = np.flatnonzero(keys == keys[act].max())[-64:]
    return np.unique(np.concatenate([[0, 1, n - 2, n - 1], first, last, rng.integers(0, n, size=k)])).astype(np.int64)


def test_meta_max_rows():
    rng = np.random.default_rng(71)
    slot = rng.integers(-40, S_MULTI_MAX + 40, size=N_MAX).astype(np.int32)   # inactive and invalid too
    check_meta(slot, S_MULTI_MAX)


def test_fused_max_rows():
    c = small_case(72, n=N_MAX, k_in=8, slices=(8,), S=S_MULTI_MAX, R=8)
    print(f"fused max rows: n={c.n} S={c.num_slots}", flush=True)
    dv = Dev(c)
    dv.fused()
    y = h16(dv.y)
    off = ~active(c)
    assert np.array_equal(y[off], dv.y_host[off]), "rows without an adapter must stay bitwise unchanged"
    sel = sample_rows(np.random.default_rng(73), c.slot, c.num_slots)
    check_y(dv, y, sel, "fused max rows")


def test_moe_max_pairs():
    """2^19 tokens x top_k 8 = 2^22 pairs over 64 experts x 128 adapters."""
    c = I.make_moe(74, T=1 << 19, H=8, E=64, top_k=8, I=8, R=8, L=128, neg_frac=0.1)
    rng = np.random.default_rng(74)
    c.lora_ids[rng.random(c.T) < 0.01] = c.L + 3          # invalid adapters
    c.topk_ids[rng.random(c.topk_ids.shape) < 0.01] = -1   # invalid experts
    assert c.T * c.top_k == N_MAX and c.E * c.L == S_MULTI_MAX
    print(f"moe max pairs: T={c.T} pairs={c.T * c.top_k} keys={c.E * c.L}", flush=True)
    out, _, ws = run_moe(c, False)
    lora = np.repeat(c.lora_ids, c.top_k)
    ex = c.topk_ids.reshape(-1)
    valid = (lora >= 0) & (lora < c.L) & (ex >= 0) & (ex < c.E)
    assert not out[~valid].any(), "pairs without a valid (adapter, expert) must be zero rows"
    assert not (out[valid] == SENTINEL).all(axis=1).any(), "a routed pair's row was never written"
    check_pair_meta(c, ws)   # sorted pairs, segments, tiles and counts, bit for bit
    sel = sample_rows(rng, O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L), c.E * c.L)
    assert_close_chunked(out, lambda p: O.case_moe_pairs(c, False, p), sel, "moe max pairs", chunk=2048)


def test_moe_w2_max_pairs():
    """The routed down-projection delta, weighted, over 2^22 pairs and 8192
    (adapter, expert) keys; unrouted rows of y unchanged bit for bit."""
    c = I.make_moe_w2(75, T=1 << 19, H=8, E=64, top_k=8, I=8, R=8, L=128, neg_frac=0.1)
    rng = np.random.default_rng(75)
    c.lora_ids[rng.random(c.T) < 0.01] = c.L + 3
    c.topk_ids[rng.random(c.topk_ids.shape) < 0.01] = c.E + 1
    assert c.T * c.top_k == N_MAX and c.E * c.L == S_MULTI_MAX
    print(f"moe w2 max pairs: T={c.T} pairs={c.T * c.top_k} keys={c.E * c.L}", flush=True)
    out, _, ws = run_w2(c, True)
    lora = np.repeat(c.lora_ids, c.top_k)
    ex = c.topk_ids.reshape(-1)
    valid = (lora >= 0) & (lora < c.L) & (ex >= 0) & (ex < c.E)
    assert np.array_equal(out[~valid], c.y[~valid]), "unrouted pairs must keep y bit for bit"
    check_pair_meta(c, ws)   # sorted pairs, segments, tiles and counts, bit for bit
    sel = sample_rows(rng, O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L), c.E * c.L)
    assert_close_chunked(out, lambda p: O.case_moe_w2_pairs(c, p, True), sel, "moe w2 max pairs", chunk=2048)
