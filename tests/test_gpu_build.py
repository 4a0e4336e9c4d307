"""GPU parity of lora_delta_fused_build (the routing metadata and the fused
delta in one call) against the fp64 oracle: every row of y within tolerance
and bitwise unchanged outside the windows and on inactive rows, and the
metadata it writes bit-exact with the oracle's (and so with
lora_meta_build's).  Decode-sized batches take the one-launch path (each
workgroup derives its tile's record from the slot array; one more writes the
metadata); larger ones take the metadata kernel, then the fused kernel."""
import numpy as np
import pytest
import torch

from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import assert_ws_ok, d32, h16
from test_gpu_dense import PATHS, Dev, check_y, small_case
from test_gpu_meta import assert_meta_matches

pytestmark = pytest.mark.gpu


@pytest.fixture(params=list(PATHS))
def path(request):
    old = B.mfma_min_rows()
    B.set_mfma_min_rows(PATHS[request.param])
    yield request.param
    B.set_mfma_min_rows(old)


def build(dv: Dev, ws=None, calls=None):
    c = dv.c
    ws = B.fused_build_workspace(c.n, c.num_slots, c.num_slices, c.max_rank, c.k_in) if ws is None else ws
    meta = B.LoraMeta.allocate(c.n, c.num_slots)
    meta.tiles.fill_(-7)   # record words a build leaves alone must not matter
    B.lora_delta_fused_build(dv.x, dv.a, dv.b, dv.scale, c.slice_sizes, dv.slot, dv.y, meta=meta,
                             offset_start=dv.offset_start, ws=ws)
    assert_ws_ok(ws, calls=calls)
    return meta, ws


BUILD = [
    dict(seed=11, n=70),                                          # one launch
    dict(seed=12, n=256, k_in=1032, slices=(520, 16), S=64, R=24),   # 256 rows, 64 slots: one launch
    dict(seed=13, n=1, k_in=8, slices=(8,), S=1, R=8),            # one row
    dict(seed=14, n=200, k_in=512, slices=(1024,), S=2, R=128, zipf=True),   # rank 128, long segments
    dict(seed=15, n=129, k_in=128, slices=(8,) * 8, S=5, R=8),    # 8 slices
    dict(seed=16, n=300, S=4, zipf=True),                         # more than 256 rows: two launches
    dict(seed=17, n=100, S=65),                                   # more than 64 slots: two launches
    dict(seed=18, n=1500, k_in=256, slices=(256,), S=7, R=16, zipf=True),   # several metadata chunks
]


@pytest.mark.parametrize("kw", BUILD, ids=[f"b{k['seed']}" for k in BUILD])
def test_build_small(kw, path):
    c = small_case(**kw)
    print(f"build small {kw} path={path}", flush=True)
    dv = Dev(c, ldy_pad=16, offset_start=8)
    meta, _ = build(dv, calls=1)
    check_y(dv, h16(dv.y), None, f"build {kw} {path}")
    assert_meta_matches(meta, c.slot, c.num_slots)


def test_build_decode_config(path):
    c = I.decode_bgmv()
    print(f"build decode config path={path}", flush=True)
    dv = Dev(c)
    meta, _ = build(dv, calls=1)
    check_y(dv, h16(dv.y), None, f"build decode {path}")
    assert_meta_matches(meta, c.slot, c.num_slots)


def test_build_equals_meta_build_then_fused():
    """The same bits as lora_meta_build followed by lora_delta_fused."""
    c = I.decode_bgmv(seed=25)
    a, b = Dev(c), Dev(c)
    a.fused()
    build(b)
    assert np.array_equal(h16(a.y), h16(b.y))


def test_build_workspace_shared_with_fused_calls():
    """One workspace through build, fused and build calls of different
    batches: every call checked in full (the tags keep the calls apart)."""
    cases = [I.decode_bgmv(seed=26), small_case(seed=27, n=90, k_in=4096, slices=(4096, 1024, 1024), S=32),
             I.decode_bgmv(seed=28), small_case(seed=29, n=256, k_in=4096, slices=(4096, 1024, 1024), S=32)]
    ws = B.fused_build_workspace(256, 32, 3, 16, 4096)
    for i, c in enumerate(cases):
        print(f"shared workspace call {i}", flush=True)
        dv = Dev(c)
        if i % 2 == 0:
            meta, _ = build(dv, ws=ws, calls=i + 1)
            assert_meta_matches(meta, c.slot, c.num_slots)
        else:
            dv.fused(ws=ws)
            assert_ws_ok(ws, calls=i + 1)
        check_y(dv, h16(dv.y), None, f"shared workspace call {i}")


def test_build_meta_counters_survive_shapes():
    """One workspace, builds of two kinds in turn: 6000 rows over 2000 slots
    (too many for the per-chunk slot table, so one workgroup assembles,
    taking a ticket) and 3000 rows over 7 slots (one assembling workgroup per
    chunk).  The larger call's flags cover the place the smaller call's
    metadata workspace starts at, so the build's counters (the ticket and the
    invalid-row count) must live where no call of any shape writes anything
    else; every call is checked in full, its counts included."""
    kw_t = dict(n=6000, k_in=64, slices=(64,), S=2000, R=8)
    kw_s = dict(n=3000, k_in=64, slices=(64,), S=7, R=8, zipf=True)
    cases = [small_case(31, **kw_t), small_case(32, **kw_s), small_case(33, **kw_t), small_case(34, **kw_s)]
    need = max(B.fused_build_workspace(c.n, c.num_slots, c.num_slices, c.max_rank, c.k_in).numel()
               for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, c in enumerate(cases):
        assert ((c.slot >= c.num_slots).any() and (c.slot < 0).any())
        print(f"counter call {i}: n={c.n} S={c.num_slots}", flush=True)
        dv = Dev(c)
        meta, _ = build(dv, ws=ws, calls=i + 1)
        assert_meta_matches(meta, c.slot, c.num_slots)
        check_y(dv, h16(dv.y), None, f"counter call {i}")


def test_build_zero_rows():
    """n == 0: only the counts are written (zero); no row is read."""
    import ctypes
    c = small_case(seed=30, n=8)
    dv = Dev(c)
    meta = B.LoraMeta.allocate(0, c.num_slots)
    meta.counts.fill_(5)
    ws = B.fused_build_workspace(8, c.num_slots, c.num_slices, c.max_rank, c.k_in)
    ss = (ctypes.c_int32 * c.num_slices)(*c.slice_sizes)
    st = B.lib().lora_delta_fused_build(dv.x.data_ptr(), c.k_in, 0, c.k_in, dv.a.data_ptr(), dv.b.data_ptr(),
                                        dv.scale.data_ptr(), c.num_slots, c.num_slices, ss, c.max_rank, None,
                                        meta.struct(), dv.y.data_ptr(), c.n_out, 0, ws.data_ptr(), ws.numel(),
                                        torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert meta.counts.cpu().tolist() == [0] * 8


def test_build_rejects_a_small_workspace():
    c = I.decode_bgmv()
    dv = Dev(c)
    need = B.fused_build_workspace(c.n, c.num_slots, c.num_slices, c.max_rank, c.k_in).numel()
    with pytest.raises(B.LoraError):
        B.lora_delta_fused_build(dv.x, dv.a, dv.b, dv.scale, c.slice_sizes, dv.slot, dv.y,
                                 ws=torch.zeros(need - 256, dtype=torch.uint8, device="cuda"))
