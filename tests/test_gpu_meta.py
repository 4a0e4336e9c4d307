"""GPU parity of lora_meta_build against the oracle: bit-exact integer
metadata (sorted rows, segment offsets, active-slot list, counts) and tile
records derived on the host from the oracle's segments."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I
from tenant_lora_serving_amd import lora as B
from gpu_util import d32

pytestmark = pytest.mark.gpu


def expected_tiles(rows, offs, sl, n):
    """Tile records from the oracle's segments: 16-row tiles, the last one
    ragged; in batches of at most 1024 rows a segment of 9..15 rows is cut
    into two tiles (ceil, floor)."""
    out = []
    for g in range(len(sl)):
        m = int(offs[g + 1] - offs[g])
        per = (m + 1) // 2 if (n <= 1024 and 8 < m < 16) else 16
        for o in range(0, m, per):
            k = min(per, m - o)
            p = int(offs[g]) + o
            out.append((int(sl[g]), p, k, m, g, o // per, rows[p:p + k].tolist()))
    return out


def check_meta(slot: np.ndarray, S: int):
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    print(f"meta case n={slot.size} S={S}", flush=True)
    meta = B.lora_meta_build(d32(slot), S)
    torch.cuda.synchronize()
    return assert_meta_matches(meta, slot, S)


def assert_meta_matches(meta, slot: np.ndarray, S: int):
    """Device metadata == the oracle's for the per-row slots, bit for bit."""
    rows, offs, sl, cnt = O.meta_build(slot, S)
    g_cnt = meta.counts.cpu().numpy()
    na, ns = int(cnt[0]), int(cnt[1])
    assert g_cnt[:4].tolist() == cnt.tolist()
    assert meta.sorted_rows.cpu().numpy()[:na].tolist() == rows.tolist()
    assert meta.seg_offsets.cpu().numpy()[:ns + 1].tolist() == offs.tolist()
    assert meta.seg_slot.cpu().numpy()[:ns].tolist() == sl.tolist()
    exp = expected_tiles(rows, offs, sl, slot.size)
    assert int(g_cnt[4]) == len(exp)
    bound = B.lib().lora_meta_max_tiles(slot.size, S)
    assert len(exp) <= bound
    tiles = meta.tiles.cpu().numpy().reshape(-1, 32)
    for t, (s, p, k, m, g, jt, rid) in enumerate(exp):
        rec = tiles[t]
        assert rec[:6].tolist() == [s, p, k, m, g, jt], (t, rec[:6])
        assert rec[8:8 + k].tolist() == rid
    for t in range(len(exp), bound):
        assert not tiles[t][:8].any(), (t, tiles[t][:8])   # unused records: zero header
    # the workspace counters are back to zero
    if meta.ws.numel() >= 8:
        assert meta.ws[:8].view(torch.int32).cpu().tolist() == [0, 0]
    return meta


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_meta_dense_configs(cfg):
    c = I.CONFIGS[cfg]()
    check_meta(c.slot, c.num_slots)


def test_meta_prefill_config():
    rng = np.random.default_rng(3)
    lens = rng.integers(64, 1025, size=16)
    slot = np.repeat(rng.integers(0, 16, size=16), lens).astype(np.int32)
    check_meta(slot, 16)


def test_meta_moe_keys_config():
    c = I.moe_gemm1()
    keys = O.moe_keys(c.topk_ids, c.lora_ids, c.E, c.L)
    check_meta(keys, c.E * c.L)


@pytest.mark.parametrize("n,S,lo", [
    (0, 4, -1), (1, 1, 0), (7, 3, -2), (63, 5, -1), (64, 2, 0), (65, 9, -1), (1023, 100, -5),
    (1024, 1024, -1), (1025, 7, -1), (2048, 1, 0), (3000, 37, -3), (5000, 8192, -10),
    (16384, 512, -40), (20000, 300, -1), (65536, 4000, -100)])
def test_meta_random(n, S, lo):
    rng = np.random.default_rng(n * 7919 + S)
    slot = rng.integers(lo, S + 3, size=n).astype(np.int32)   # includes invalid slots >= S
    check_meta(slot, S)


def test_meta_degenerate():
    check_meta(np.full(3000, -1, np.int32), 8)                 # nothing active
    check_meta(np.full(1500, 9, np.int32), 8)                  # everything invalid
    check_meta(np.full(5000, 3, np.int32), 8)                  # one segment of 5000 rows
    check_meta(np.arange(1024, dtype=np.int32)[::-1].copy(), 1024)   # all distinct, reversed
    check_meta(np.random.default_rng(0).integers(0, 1 << 20, 900).astype(np.int32), 1 << 20)


def test_meta_reuse_buffers_and_determinism():
    rng = np.random.default_rng(5)
    slot = rng.integers(-1, 40, size=4000).astype(np.int32)
    m = B.LoraMeta.allocate(4000, 40)
    for _ in range(3):
        B.lora_meta_build(d32(slot), 40, m)
    torch.cuda.synchronize()
    rows, offs, sl, cnt = O.meta_build(slot, 40)
    assert m.sorted_rows.cpu().numpy()[:cnt[0]].tolist() == rows.tolist()
    assert m.ws[:8].view(torch.int32).cpu().tolist() == [0, 0]


def test_meta_assembly_paths_share_a_workspace():
    """Builds that assemble in a second launch (the [chunk][slot] table fits)
    and builds whose last workgroup assembles alone (8192 slots), one after
    another on one workspace: each matches the oracle and leaves the
    workspace counters at zero for the next."""
    # (70000, 5): 69 chunks, past the split build's limit, so its table path assembles alone
    shapes = [(4000, 40), (5000, 8192), (20000, 300), (3000, 8192), (70000, 5), (4000, 40)]
    wsb = max(int(B.lib().lora_meta_workspace_bytes(n, S)) for n, S in shapes)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for i, (n, S) in enumerate(shapes):
        rng = np.random.default_rng(300 + i)
        slot = rng.integers(-2, S + 2, size=n).astype(np.int32)
        print(f"meta shared-ws case n={n} S={S}", flush=True)
        m = B.LoraMeta.allocate(n, S)
        m.ws = ws
        B.lora_meta_build(d32(slot), S, m)
        torch.cuda.synchronize()
        assert_meta_matches(m, slot, S)
