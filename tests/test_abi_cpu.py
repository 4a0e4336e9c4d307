"""CPU-only checks of the C ABI: the built library loads, exports every
function include/lora.h declares, and rejects bad arguments on the host with
the documented status codes before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from tenant_lora_serving_amd import lora as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")

OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"})


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("liblora.so is not built (python -m tenant_lora_serving_amd.build)")
    return B.lib()


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for f in ["lora_meta_build", "lora_shrink", "lora_expand", "lora_delta_fused",
              "moe_lora_gemm1_delta", "moe_lora_w2_delta", "lora_meta_from_offsets"]:
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(B.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(raw, f)]
    assert not missing, missing
    assert sorted(B.EXPORTED) == declared_functions()


def test_library_exports_no_other_c_symbols(L):
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm is not available")
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    # unmangled text symbols are the C entry points (the host build's launcher
    # stand-ins add stub_* and the two HIP runtime calls it replaces)
    c_syms = {s for s in syms if not s.startswith(("_Z", "stub_", "hipGetDevice", "hipStreamGetDevice"))}
    assert sorted(c_syms) == declared_functions()


def test_tile_bound_and_workspace_sizes(L):
    assert L.lora_meta_max_tiles(0, 4) == 0
    assert L.lora_meta_max_tiles(8, 4) == 5          # ceil(8/16) + min(8, 4) + 0 split segments
    assert L.lora_meta_max_tiles(256, 32) == 64       # min(16 + 32 + 28, 32 + 32): 9..15-row segments split
    assert L.lora_meta_max_tiles(6947, 16) == 451     # 435 + 16: no split past 1024 rows
    assert L.lora_meta_max_tiles(1024, 1024) == 1024  # capped at n
    # the bound holds for the worst partitions: every segment split (9 or 15 rows),
    # every segment one row, one long segment, and past 1024 rows (no split)
    for n, S, lens in [(9 * 40, 40, [9] * 40), (15 * 33, 33, [15] * 33), (50, 50, [1] * 50),
                       (5000, 1, [5000]), (16 * 7 + 9 * 5, 12, [16] * 7 + [9] * 5),
                       (9 * 113, 113, [9] * 113), (9 * 200, 200, [9] * 200)]:
        tiles = sum(2 if (n <= 1024 and 8 < t < 16) else -(-t // 16) for t in lens)
        assert tiles <= L.lora_meta_max_tiles(n, S), (n, S, tiles)
    assert L.lora_meta_workspace_bytes(1024, 8) == 0  # one chunk needs none
    assert L.lora_meta_workspace_bytes(1025, 8) > 0
    assert L.lora_meta_workspace_bytes(5000, 9000) == 0  # unsupported -> 0
    assert L.lora_fused_workspace_bytes(256, 32, 3, 16, 4096) > 0
    assert L.lora_fused_workspace_bytes(256, 32, 3, 12, 4096) == 0  # rank not a multiple of 8
    assert L.moe_lora_workspace_bytes(2048, 8, 64, 8, 16, 4096) > 0
    # one shrink slice over I = 1408: smaller than gemm1's two over H = 4096
    w2 = L.moe_lora_w2_workspace_bytes(2048, 8, 64, 8, 16, 1408)
    assert 0 < w2 < L.moe_lora_workspace_bytes(2048, 8, 64, 8, 16, 4096)
    assert L.moe_lora_w2_workspace_bytes(2048, 8, 64, 8, 12, 1408) == 0


def _meta(ptr=0x10000):
    return B._MetaStruct(ptr, ptr, ptr, ptr, ptr)


def test_meta_build_validation(L):
    m = _meta()
    assert L.lora_meta_build(0x1000, -1, 4, m, None, 0, None) == EINVAL
    assert L.lora_meta_build(0x1000, 8, 0, m, None, 0, None) == EINVAL
    assert L.lora_meta_build(None, 8, 4, m, None, 0, None) == EINVAL
    assert L.lora_meta_build(0x1000, 8, 4, B._MetaStruct(0, 0, 0, 0, 0), None, 0, None) == EINVAL
    # two chunks need a workspace
    assert L.lora_meta_build(0x1000, 2000, 4, m, None, 0, None) == EWS
    assert L.lora_meta_build(0x1000, 2000, 4, m, 0x2000, 16, None) == EWS
    # several chunks support at most 8192 slots
    assert L.lora_meta_build(0x1000, 2000, 9000, m, 0x2000, 1 << 30, None) == EUNSUP


def test_shrink_validation(L):
    m = _meta()
    a = dict(x=0x1000, ldx=256, n=8, k_in=256, a=0x2000, sc=0x3000, S=4, L=1, R=8, xa=0x4000)

    def call(**kw):
        v = dict(a, **kw)
        return L.lora_shrink(v["x"], v["ldx"], v["n"], v["k_in"], v["a"], v["sc"], v["S"], v["L"],
                             v["R"], m, v["xa"], None)
    assert call(k_in=260) == EINVAL          # not a multiple of 8
    assert call(ldx=128) == EINVAL           # ldx < k_in
    assert call(x=0x1008) == EINVAL          # x not 16-byte aligned
    assert call(R=12) == EUNSUP
    assert call(R=136) == EUNSUP
    assert call(L=9) == EINVAL
    assert call(L=0) == EINVAL
    assert call(xa=None) == EINVAL
    assert call(n=0) == OK                   # nothing to do, nothing launched


def test_expand_and_fused_validation(L):
    m = _meta()
    ss = (ctypes.c_int32 * 2)(256, 128)
    bad = (ctypes.c_int32 * 2)(256, 100)
    assert L.lora_expand(0x1000, 0x2000, 4, 2, bad, 8, 8, m, 0x3000, 384, 0, 1, None) == EINVAL
    assert L.lora_expand(0x1000, 0x2000, 4, 2, ss, 8, 8, m, 0x3000, 376, 0, 1, None) == EINVAL  # ldy < N
    assert L.lora_expand(0x1000, 0x2000, 4, 2, ss, 8, 8, m, 0x3000, 392, 12, 1, None) == EINVAL
    assert L.lora_expand(0x1000, 0x2000, 4, 2, ss, 8, 8, m, 0x3000, 392, 16, 1, None) == EINVAL
    assert L.lora_expand(0x1000, 0x2000, 4, 2, ss, 8, 0, m, 0x3000, 384, 0, 1, None) == OK
    ws_need = L.lora_fused_workspace_bytes(8, 4, 2, 8, 256)
    args = [0x1000, 256, 8, 256, 0x2000, 0x3000, 0x4000, 4, 2, ss, 8, m, 0x5000, 384, 0]
    assert L.lora_delta_fused(*args, 0x6000, ws_need - 1, None) == EWS
    assert L.lora_delta_fused(*args, None, ws_need, None) == EWS
    args0 = list(args)
    args0[2] = 0
    assert L.lora_delta_fused(*args0, 0x6000, 1 << 20, None) == OK


def test_build_validation(L):
    m = _meta()
    ss = (ctypes.c_int32 * 2)(256, 128)
    need = L.lora_fused_workspace_bytes(8, 4, 2, 8, 256) + L.lora_meta_workspace_bytes(8, 4)
    args = [0x1000, 256, 8, 256, 0x2000, 0x3000, 0x4000, 4, 2, ss, 8, 0x7000, m, 0x5000, 384, 0]
    assert L.lora_delta_fused_build(*args, 0x6000, need - 1, None) == EWS
    bad = list(args)
    bad[11] = None                      # rows but no slot array
    assert L.lora_delta_fused_build(*bad, 0x6000, need, None) == EINVAL
    bad = list(args)
    bad[12] = _meta(0)                  # nowhere to write the metadata
    assert L.lora_delta_fused_build(*bad, 0x6000, need, None) == EINVAL
    bad = list(args)
    bad[10] = 12                        # rank not a multiple of 8
    assert L.lora_delta_fused_build(*bad, 0x6000, need, None) == EUNSUP


def test_moe_validation(L):
    base = dict(x=0x1000, ldx=4096, T=16, H=4096, wa=0x2000, lsa=16 * 4096, wb=0x3000, lsb=1408 * 16,
                shared=0, topk=0x4000, top_k=8, lora=0x5000, E=64, L=8, R=16, I=1408, out=0x6000)
    need = L.moe_lora_workspace_bytes(16, 8, 64, 8, 16, 4096)

    def call(ws=0x7000, wsb=need, **kw):
        v = dict(base, **kw)
        return L.moe_lora_gemm1_delta(v["x"], v["ldx"], v["T"], v["H"], v["wa"], v["lsa"], v["wb"],
                                      v["lsb"], v["shared"], v["topk"], v["top_k"], v["lora"], v["E"],
                                      v["L"], v["R"], v["I"], 1.0, v["out"], ws, wsb, None)
    assert call(I=1404) == EINVAL
    assert call(R=20) == EUNSUP
    assert call(H=4100) == EINVAL
    assert call(lsa=7) == EINVAL
    assert call(wa=None) == EINVAL
    assert call(wsb=need - 1) == EWS
    assert call(top_k=0) == EINVAL


def test_meta_from_offsets_validation(L):
    m = _meta()
    assert L.lora_meta_from_offsets(None, 64, 0x2000, 100, 48, m, None, 0, None) == EINVAL
    assert L.lora_meta_from_offsets(0x1000, 64, None, 100, 48, m, None, 0, None) == EINVAL
    assert L.lora_meta_from_offsets(0x1000, -1, 0x2000, 100, 48, m, None, 0, None) == EINVAL
    assert L.lora_meta_from_offsets(0x1000, 64, 0x2000, -5, 48, m, None, 0, None) == EINVAL
    assert L.lora_meta_from_offsets(0x1000, 64, 0x2000, 100, 0, m, None, 0, None) == EINVAL
    assert L.lora_meta_from_offsets(0x1000, 64, 0x2000, 100, 48, _meta(0), None, 0, None) == EINVAL
    assert L.lora_meta_from_offsets(0x1000, 64, 0x2000, 5000, 48, m, None, 0, None) == EWS
    assert L.lora_meta_from_offsets(0x1000, 64, 0x2000, 5000, 9000, m, 0x3000, 1 << 20, None) == EUNSUP


def test_moe_w2_validation(L):
    base = dict(x=0x1000, ldx=1408, T=16, I=1408, wa=0x2000, lsa=16 * 1408, wb=0x3000, lsb=4096 * 16,
                topk=0x4000, top_k=8, lora=0x5000, wt=0x8000, E=64, L=8, R=16, H=4096, y=0x6000,
                ldy=4096)
    need = L.moe_lora_w2_workspace_bytes(16, 8, 64, 8, 16, 1408)

    def call(ws=0x7000, wsb=need, **kw):
        v = dict(base, **kw)
        return L.moe_lora_w2_delta(v["x"], v["ldx"], v["T"], v["I"], v["wa"], v["lsa"], v["wb"], v["lsb"],
                                   v["topk"], v["top_k"], v["lora"], v["wt"], v["E"], v["L"], v["R"],
                                   v["H"], 1.0, v["y"], v["ldy"], 0, ws, wsb, None)
    assert call(I=1404) == EINVAL
    assert call(ldx=1400) == EINVAL
    assert call(R=20) == EUNSUP
    assert call(H=4100) == EINVAL
    assert call(ldy=4000) == EINVAL
    assert call(y=0x6008) == EINVAL          # y not 16-byte aligned
    assert call(wt=0x8002) == EINVAL         # weights not float aligned
    assert call(lsb=7) == EINVAL
    assert call(wb=None) == EINVAL
    assert call(topk=None) == EINVAL
    assert call(wsb=need - 1) == EWS
    assert call(ws=None) == EWS
    assert call(top_k=0) == EINVAL
    assert call(E=0) == EINVAL


def test_status_strings(L):
    for s in (OK, EINVAL, EUNSUP, EWS, -4, 99):
        assert isinstance(L.lora_status_string(s), bytes)


def test_moe_meta_layout(L):
    off = (ctypes.c_size_t * 5)()
    assert L.moe_lora_meta_layout(2048, 8, 64, 8, off) == OK
    n, S = 2048 * 8, 64 * 8
    up = lambda v: (v + 255) // 256 * 256   # noqa: E731
    # counts at byte 0; the header line (counts, control line) is 256 bytes
    assert list(off) == [0, 256, 256 + up(4 * n), 256 + up(4 * n) + up(4 * (min(n, S) + 1)),
                         256 + up(4 * n) + up(4 * (min(n, S) + 1)) + up(4 * min(n, S))]
    assert B.MOE_CTL_OFFSET + 12 <= 256 and B.MOE_CTL_OFFSET >= 32   # clear of the 8 counts
    # the tiles fit every MoE workspace of that routing, gemm1 (either form) or w2
    tiles_end = off[4] + 4 * 32 * L.lora_meta_max_tiles(n, S)
    assert tiles_end <= L.moe_lora_workspace_bytes(2048, 8, 64, 8, 16, 4096)
    assert tiles_end <= L.moe_lora_w2_workspace_bytes(2048, 8, 64, 8, 8, 8)
    assert L.moe_lora_meta_layout(-1, 8, 64, 8, off) == EINVAL
    assert L.moe_lora_meta_layout(16, 0, 64, 8, off) == EINVAL
    assert L.moe_lora_meta_layout(16, 8, 64, 8, None) == EINVAL


def test_mfma_threshold_is_per_thread(L):
    import threading
    default = L.lora_mfma_min_rows()
    seen = {}

    def other():
        seen["before"] = L.lora_mfma_min_rows()
        L.lora_set_mfma_min_rows(3)
        seen["after"] = L.lora_mfma_min_rows()

    L.lora_set_mfma_min_rows(7)
    t = threading.Thread(target=other)
    t.start()
    t.join()
    try:
        assert L.lora_mfma_min_rows() == 7          # the other thread's setting is not seen here
        assert seen == {"before": default, "after": 3}
        L.lora_set_mfma_min_rows(0)
        assert L.lora_mfma_min_rows() == default    # 0 drops the override
    finally:
        L.lora_set_mfma_min_rows(0)


def test_noalloc_rejects_oversize_before_any_launch(L):
    m = _meta()
    ss = (ctypes.c_int32 * 1)(1024)
    # 4096 rows, rank 64, k_in 4096: the workspace would exceed the fixed buffer
    need = L.lora_fused_workspace_bytes(4096, 16, 1, 64, 4096)
    assert need > B.NOALLOC_SCRATCH_BYTES
    args = [0x1000, 4096, 4096, 4096, 0x2000, 0x3000, 0x4000, 16, 1, ss, 64, m, 0x5000, 1024, 0, None]
    assert L.lora_delta_fused_noalloc(*args) == -5
    assert L.lora_status_string(-5) != L.lora_status_string(99)
    # the same argument checks as lora_delta_fused come first
    bad = list(args)
    bad[3] = 4100
    assert L.lora_delta_fused_noalloc(*bad) == EINVAL
    zero = list(args)
    zero[2] = 0
    zero[10] = 16
    assert L.lora_delta_fused_noalloc(*zero) == OK   # nothing to do: no device touched
