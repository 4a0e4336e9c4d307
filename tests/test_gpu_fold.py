"""GPU parity of the expert-sorted fold and the router fold: the metadata
lora_meta_from_offsets builds on the device from the expert_offsets prefix sum
equals, bit for bit, the oracle's metadata for the rows the oracle's work
items assign to each adapted expert; the folded output matches the oracle's
fold of each work item's pair over its block."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close, assert_close_chunked, assert_ws_ok, bf64, d16, d32, h16
from test_gpu_meta import assert_meta_matches

pytestmark = pytest.mark.gpu


def row_slots(c: I.ExpertFoldCase):
    """Per sorted row, the pool slot the oracle's work items give it (-1: none)."""
    slot = np.full(c.n, -1, np.int32)
    for e, r0, nr in O.expert_workitems(c.expert_offsets, c.adapted):
        slot[r0:r0 + nr] = c.expert_slot[e]
    return slot


def offsets_dev(off: np.ndarray) -> torch.Tensor:
    return d32(np.ascontiguousarray(off, dtype=np.uint32).view(np.int32))


def check_fold(c: I.ExpertFoldCase, what=""):
    print(f"fold case n={c.n} E={c.E} k_in={c.k_in} n_out={c.n_out} R={c.R} slots={c.num_slots} {what}",
          flush=True)
    y = d16(c.y)
    meta = B.lora_meta_from_offsets(offsets_dev(c.expert_offsets), d32(c.expert_slot), c.n, c.num_slots)
    ws = B.fused_workspace(c.n, c.num_slots, 1, c.R, c.k_in)
    B.lora_delta_fused(d16(c.x), d16(c.a_pool), d16(c.b_pool), d32(c.scale), (c.n_out,), meta, y, ws=ws)
    assert_ws_ok(ws, calls=1)
    assert_meta_matches(meta, row_slots(c), c.num_slots)
    out = h16(y)
    slot = row_slots(c)
    keep = (slot < 0) | (slot >= c.num_slots)
    assert np.array_equal(out[keep], c.y[keep]), "rows outside the adapted blocks changed"
    items = O.expert_workitems(c.expert_offsets, c.adapted)
    orc = O.fold_sorted(c.x, c.k_in, c.y, items, c.expert_slot, c.a_pool, c.b_pool, c.scale,
                        c.num_slots, (c.n_out,), c.R)
    rows = np.flatnonzero((slot >= 0) & (slot < c.num_slots))
    return assert_close(bf64(out[rows]), orc[rows], f"fold {what}")


@pytest.mark.parametrize("seed,kw", [
    (1, dict(T=40, top_k=3, E=6, k_in=72, n_out=40, R=8)),
    (2, dict(T=300, top_k=4, E=5, k_in=520, n_out=1096, R=16)),     # long blocks: MFMA tiles
    (3, dict(T=1500, top_k=2, E=24, k_in=136, n_out=64, R=32)),     # several meta chunks
    (4, dict(T=50, top_k=2, E=300, k_in=64, n_out=24, R=8, adapted_frac=0.3)),  # many empty experts
])
def test_fold_small(seed, kw):
    check_fold(I.make_expert_fold(seed, **kw), what=f"seed={seed}")


def test_fold_invalid_and_unused_slots():
    c = I.make_expert_fold(5, T=80, top_k=3, E=8, k_in=64, n_out=32, R=8, adapted_frac=0.75)
    # a slot past the pool: its rows are counted invalid and keep their output
    c.expert_slot[int(c.adapted[0])] = c.num_slots + 3
    check_fold(c, what="invalid slot")


def test_fold_rows_past_the_offsets_are_untouched():
    c = I.make_expert_fold(6, T=60, top_k=2, E=5, k_in=64, n_out=32, R=8, adapted_frac=1.0)
    c.expert_offsets = np.minimum(c.expert_offsets, c.n - 17).astype(np.uint32)  # last 17 rows in no block
    check_fold(c, what="tail")


def test_router_fold_full():
    c = I.router_fold()
    print(f"router fold n={c.n} hidden={c.k_in} E={c.n_out}", flush=True)
    g = d16(c.y)
    ws = B.fused_workspace(c.n, 1, 1, c.R, c.k_in)
    B.apply_router_lora(d16(c.x), g, d16(c.a_pool[0, 0]), d16(c.b_pool[0]), float(c.scale[0]), ws=ws)
    assert_ws_ok(ws, calls=1)
    orc = O.fold_sorted(c.x, c.k_in, c.y, [(0, 0, c.n)], c.expert_slot, c.a_pool, c.b_pool, c.scale,
                        1, (c.n_out,), c.R)
    assert_close(bf64(h16(g)), orc, "router")


def test_expert_fold_full():
    c = I.expert_fold()
    y = d16(c.y)
    meta = B.LoraMeta.allocate(c.n, c.num_slots)
    ws = B.fused_workspace(c.n, c.num_slots, 1, c.R, c.k_in)
    B.apply_expert_lora_sorted(d16(c.x), y, offsets_dev(c.expert_offsets), d32(c.expert_slot),
                               d16(c.a_pool), d16(c.b_pool), d32(c.scale), meta=meta, ws=ws)
    assert_ws_ok(ws, calls=1)
    assert_meta_matches(meta, row_slots(c), c.num_slots)
    out = h16(y)
    slot = row_slots(c)
    assert np.array_equal(out[slot < 0], c.y[slot < 0])
    # the oracle folds every work item's pair over its whole block
    items = O.expert_workitems(c.expert_offsets, c.adapted)
    assert len(items) > 0
    orc = O.fold_sorted(c.x, c.k_in, c.y, items, c.expert_slot, c.a_pool, c.b_pool, c.scale,
                        c.num_slots, (c.n_out,), c.R)
    rows = np.flatnonzero(slot >= 0)
    assert_close_chunked(out, lambda r: orc[r], rows, "expert fold full", chunk=2048)
