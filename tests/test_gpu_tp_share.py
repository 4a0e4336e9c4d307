"""The one-GPU share of tensor-parallel (S-LoRA) LoRA layers, at real shard
shapes, against the fp64 oracle of the unsharded layer.

Column parallel (vLLM fully_sharded_layers.py, _mcp_apply): A is split along
the rank, each shard's shrink gives R/tp rank columns, the all-gather joins
them, and each rank expands into its own output columns of every slice.
Row parallel (RowParallelLinearWithShardedLoRA.apply): x and A are split
along k, the all-reduce sums the shards' xa, and rank r expands its block of
B rows at offset_start = r * N / tp of the full-width output.

The collectives are stand-ins (a concatenation and a sum over the shards on
the one GPU); every shard's shrink and expand is the library's."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close, bf64, d16, d32, h16

pytestmark = pytest.mark.gpu


def column_parallel(c: I.DenseCase, tp: int):
    """Returns the full-width output assembled from the tp ranks' local outputs."""
    R, rs = c.max_rank, c.max_rank // tp
    meta = B.lora_meta_build(d32(c.slot), c.num_slots)
    x, sc = d16(c.x), d32(c.scale)
    # each rank's shrink on its rank shard of A; the all-gather joins the columns
    xa = torch.cat([B.lora_shrink(x, d16(np.ascontiguousarray(c.a_pool[:, :, r * rs:(r + 1) * rs])), sc, meta)
                    for r in range(tp)], dim=2).contiguous()
    assert xa.shape == (c.num_slices, c.n, R)
    off = np.concatenate([[0], np.cumsum(c.slice_sizes)])
    out = np.empty((c.n, c.n_out), np.uint16)
    for r in range(tp):
        # rank r owns columns [r*w/tp, (r+1)*w/tp) of every slice
        cols = np.concatenate([np.arange(off[l] + r * w // tp, off[l] + (r + 1) * w // tp)
                               for l, w in enumerate(c.slice_sizes)])
        b_sh = d16(np.ascontiguousarray(c.b_pool[:, cols, :]))
        y_loc = d16(np.ascontiguousarray(c.y[:, cols]))
        B.lora_expand(xa, b_sh, [w // tp for w in c.slice_sizes], meta, y_loc)
        torch.cuda.synchronize()
        out[:, cols] = h16(y_loc)
    return out


def row_parallel(c: I.DenseCase, tp: int):
    assert c.num_slices == 1
    ks, ns = c.k_in // tp, c.n_out // tp
    meta = B.lora_meta_build(d32(c.slot), c.num_slots)
    x, sc = d16(c.x), d32(c.scale)
    # each rank's shrink over its k shard (a column view of x); the all-reduce sums them
    xa = None
    for r in range(tp):
        part = B.lora_shrink(x[:, r * ks:(r + 1) * ks], d16(np.ascontiguousarray(c.a_pool[..., r * ks:(r + 1) * ks])),
                             sc, meta)
        xa = part if xa is None else xa + part
    y = d16(c.y)
    for r in range(tp):
        b_sh = d16(np.ascontiguousarray(c.b_pool[:, r * ns:(r + 1) * ns, :]))
        B.lora_expand(xa, b_sh, [ns], meta, y, offset_start=r * ns)
    torch.cuda.synchronize()
    return h16(y)


def check(c, out, what):
    print(f"tp share {what} n={c.n} k_in={c.k_in} N={c.n_out} R={c.max_rank}", flush=True)
    act = (c.slot >= 0) & (c.slot < c.num_slots)
    assert np.array_equal(out[~act], c.y[~act])
    rows = np.flatnonzero(act)
    assert_close(bf64(out[rows]), O.case_fused_rows(c, rows), what)


@pytest.mark.parametrize("tp", [2, 4, 8])
def test_column_parallel_prefill_shape(tp):
    # gate_up of an 8B-class model: k_in 4096, two slices of 14336, rank 64
    # (shards of 32, 16, 8 ranks and 7168 .. 1792 columns per slice)
    c = I.make_dense(31, n=384, k_in=4096, slice_sizes=(14336, 14336), num_slots=4, max_rank=64,
                     slot_kind="uniform", scale_fixed=2.0)
    check(c, column_parallel(c, tp), f"column tp={tp}")


def test_column_parallel_decode_qkv():
    # the decode QKV batch at tp = 2: rank shards of 8, slices 2048 / 512 / 512
    c = I.decode_bgmv()
    check(c, column_parallel(c, 2), "column tp=2 decode")


@pytest.mark.parametrize("tp", [2, 4, 8])
def test_row_parallel_down_proj_shape(tp):
    # down projection: k_in 14336 split over the ranks, N 4096, decode routing
    c = I.make_dense(32, n=256, k_in=14336, slice_sizes=(4096,), num_slots=32, max_rank=16,
                     rank_choices=[8, 16], slot_kind="zipf", neg_frac=0.05, scale_num=32.0)
    check(c, row_parallel(c, tp), f"row tp={tp}")
