"""lora_delta_fused_noalloc -- the fused delta on the library's own fixed
device buffer, for callers that cannot allocate -- against lora_delta_fused
with a caller-given workspace: the same kernels, so the same bits, and both
within the oracle's tolerance.  Two calls in a row on the one buffer, the
second with a smaller batch (it finds the first call's partials there and
must not take them); then the first shape again with new inputs."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_close_chunked, assert_ws_ok, d16, d32, h16

pytestmark = pytest.mark.gpu


def both(c):
    """(noalloc result, workspace result) as bf16 bits, from the same inputs."""
    meta = B.lora_meta_build(d32(c.slot), c.num_slots)
    x, a, b, sc = d16(c.x), d16(c.a_pool), d16(c.b_pool), d32(c.scale)
    y_na, y_ws = d16(c.y), d16(c.y)
    print(f"noalloc call n={c.n} S={c.num_slots} k_in={c.k_in} N={c.n_out} R={c.max_rank}", flush=True)
    B.lora_delta_fused_noalloc(x, a, b, sc, c.slice_sizes, meta, y_na)
    ws = B.fused_workspace(c.n, c.num_slots, c.num_slices, c.max_rank, c.k_in)
    B.lora_delta_fused(x, a, b, sc, c.slice_sizes, meta, y_ws, ws=ws)
    assert_ws_ok(ws, calls=1)
    return h16(y_na), h16(y_ws)


def test_noalloc_matches_fused_on_consecutive_calls():
    big = I.decode_bgmv(seed=51)
    small = I.make_dense(52, n=40, k_in=1032, slice_sizes=(64, 32), num_slots=5, max_rank=24,
                         rank_choices=[12, 24], slot_kind="uniform_neg", scale_num=48.0)
    big2 = I.decode_bgmv(seed=53)
    need = int(B.lib().lora_fused_workspace_bytes(big.n, big.num_slots, big.num_slices, big.max_rank, big.k_in))
    assert need <= B.NOALLOC_SCRATCH_BYTES
    for c in (big, small, big2):
        got, ref = both(c)
        assert np.array_equal(got, ref), "noalloc and workspace calls differ"
        act = (c.slot >= 0) & (c.slot < c.num_slots)
        assert np.array_equal(got[~act], c.y[~act])
        assert_close_chunked(got, lambda r: O.case_fused_rows(c, r), np.flatnonzero(act),
                             f"noalloc n={c.n}")


def test_noalloc_rejects_a_call_larger_than_its_buffer():
    c = I.make_dense(54, n=4096, k_in=4096, slice_sizes=(1024,), num_slots=16, max_rank=64,
                     slot_kind="uniform", scale_fixed=1.0)
    need = int(B.lib().lora_fused_workspace_bytes(c.n, c.num_slots, c.num_slices, c.max_rank, c.k_in))
    assert need > B.NOALLOC_SCRATCH_BYTES
    meta = B.lora_meta_build(d32(c.slot), c.num_slots)
    y = d16(c.y)
    with pytest.raises(B.LoraError) as ei:
        B.lora_delta_fused_noalloc(d16(c.x), d16(c.a_pool), d16(c.b_pool), d32(c.scale), c.slice_sizes,
                                   meta, y)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    assert np.array_equal(h16(y), c.y)          # nothing was launched
