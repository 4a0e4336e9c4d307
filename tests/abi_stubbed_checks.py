"""What the C entry points hand to their launchers (host-only build).

Run only against the host build of the C ABI whose launchers are the stubs in
abi_host_stubs.cpp (test_sanitizers_cpu.py builds it with AddressSanitizer
and UndefinedBehaviorSanitizer and runs this file with the sanitizer runtime
preloaded); the file name keeps plain pytest runs from collecting it.  The
stubs count launches and keep the sizes and device addresses each launcher
was given, so these checks cover the host layer the GPU tests cannot see
directly: a rejected call launches nothing, and an accepted one passes the
workspace regions its documented layout names.
"""
import ctypes
import os

import pytest

from tenant_lora_serving_amd import lora as B

META_DENSE, META_MOE, META_BLOCKS, SHRINK, EXPAND, FUSED, MOE, MOE_W2, SCRATCH = range(9)
OK, EINVAL, EUNSUP, EWS, ESCRATCH = 0, -1, -2, -3, -5


@pytest.fixture(scope="module")
def L():
    path = os.environ.get("TL_STUBBED_LORA_LIB")
    if not path:
        pytest.skip("needs the host build of the C ABI with stub launchers")
    L = B.lib()
    assert B.LIB_PATH == path
    raw = ctypes.CDLL(path)
    for f in ("stub_calls", "stub_value", "stub_scratch_address"):
        getattr(raw, f).restype = ctypes.c_longlong
    raw.stub_calls.argtypes = [ctypes.c_int]
    raw.stub_value.argtypes = [ctypes.c_int, ctypes.c_int]
    L.raw = raw
    return L


@pytest.fixture(autouse=True)
def reset(L):
    L.raw.stub_reset()


def calls(L):
    return [L.raw.stub_calls(k) for k in range(9)]


def val(L, kind, i):
    return L.raw.stub_value(kind, i)


def meta(base):
    return B._MetaStruct(base, base + 0x10000, base + 0x20000, base + 0x30000, base + 0x40000)


def test_rejected_calls_launch_nothing(L):
    m = meta(0x100000)
    ss = (ctypes.c_int32 * 3)(4096, 1024, 1024)
    args = [0x1000, 4096, 256, 4096, 0x2000, 0x3000, 0x4000, 32, 3, ss, 16, m, 0x5000, 6144, 0]
    need = L.lora_fused_workspace_bytes(256, 32, 3, 16, 4096)
    assert L.lora_delta_fused(*args, 0x9000, need - 1, None) == EWS
    bad = list(args)
    bad[1] = 4000                                   # ldx < k_in
    assert L.lora_delta_fused(*bad, 0x9000, need, None) == EINVAL
    bad = list(args)
    bad[10] = 12                                    # rank not a multiple of 8
    assert L.lora_delta_fused(*bad, 0x9000, need, None) == EUNSUP
    assert L.lora_meta_build(0x1000, 2000, 4, m, None, 0, None) == EWS
    big = (ctypes.c_int32 * 1)(1024)
    assert L.lora_delta_fused_noalloc(0x1000, 4096, 4096, 4096, 0x2000, 0x3000, 0x4000, 16, 1, big, 64, m,
                                      0x5000, 1024, 0, None) == ESCRATCH
    assert calls(L) == [0] * 9


def test_fused_call_passes_its_workspace_and_plan(L):
    m = meta(0x100000)
    ss = (ctypes.c_int32 * 3)(4096, 1024, 1024)
    need = L.lora_fused_workspace_bytes(256, 32, 3, 16, 4096)
    assert L.lora_delta_fused(0x1000, 4096, 256, 4096, 0x2000, 0x3000, 0x4000, 32, 3, ss, 16, m, 0x5000, 6144, 0,
                              0x9000, need, None) == OK
    assert calls(L) == [0, 0, 0, 0, 0, 1, 0, 0, 0]
    assert [val(L, FUSED, i) for i in range(3)] == [256, 4096, 6144]
    assert val(L, FUSED, 3) == 0x100000 + 0x40000           # tiles
    assert val(L, FUSED, 4) == 0x100000 + 0x30000           # counts
    assert val(L, FUSED, 5) == L.lora_meta_max_tiles(256, 32)
    assert val(L, FUSED, 6) == need                         # the plan the size query describes
    assert val(L, FUSED, 7) == 0x9000
    assert val(L, FUSED, 8) == L.lora_mfma_min_rows()


def test_noalloc_call_runs_on_the_fixed_buffer(L):
    m = meta(0x100000)
    ss = (ctypes.c_int32 * 3)(4096, 1024, 1024)
    for n in (256, 64):
        L.raw.stub_reset()
        assert L.lora_delta_fused_noalloc(0x1000, 4096, n, 4096, 0x2000, 0x3000, 0x4000, 32, 3, ss, 16, m,
                                          0x5000, 6144, 0, None) == OK
        assert calls(L)[FUSED] == 1 and calls(L)[SCRATCH] == 1
        assert val(L, FUSED, 7) == L.raw.stub_scratch_address()
        assert val(L, FUSED, 6) == L.lora_fused_workspace_bytes(n, 32, 3, 16, 4096) <= B.NOALLOC_SCRATCH_BYTES


def test_meta_build_carves_its_workspace(L):
    m = meta(0x100000)
    n, S = 3000, 40
    need = L.lora_meta_workspace_bytes(n, S)
    assert need > 0
    assert L.lora_meta_build(0x1000, n, S, m, 0x200000, need, None) == OK
    assert calls(L)[META_DENSE] == 1
    assert val(L, META_DENSE, 5) == L.lora_meta_max_tiles(n, S)
    ws = [val(L, META_DENSE, i) for i in range(6, 10)]       # ctl, rows, keys, offlen
    assert ws[0] == 0x200000
    assert all(0x200000 <= a < 0x200000 + need for a in ws)
    assert ws == sorted(ws) and len(set(ws)) == 4
    assert [val(L, META_DENSE, 10), val(L, META_DENSE, 11)] == [n, S]


def moe_args(T=64, top_k=8, E=64, L_=8, R=16, H=4096, I_=1408, shared=0):
    return dict(T=T, top_k=top_k, E=E, L=L_, R=R, H=H, I=I_, shared=shared)


def test_moe_calls_use_the_documented_layout(L):
    a = moe_args()
    off = (ctypes.c_size_t * 5)()
    assert L.moe_lora_meta_layout(a["T"], a["top_k"], a["E"], a["L"], off) == OK
    need = L.moe_lora_workspace_bytes(a["T"], a["top_k"], a["E"], a["L"], a["R"], a["H"])
    ws = 0x400000
    st = L.moe_lora_gemm1_delta(0x1000, a["H"], a["T"], a["H"], 0x2000, a["R"] * a["H"], 0x3000,
                                a["I"] * a["R"], 0, 0x4000, a["top_k"], 0x5000, a["E"], a["L"], a["R"], a["I"],
                                1.0, 0x6000, ws, need, None)
    assert st == OK
    assert calls(L) == [0, 1, 0, 0, 0, 0, 1, 0, 0]
    n, S = a["T"] * a["top_k"], a["E"] * a["L"]
    got = [val(L, META_MOE, i) - ws for i in (3, 0, 1, 2, 4)]      # counts, sorted, segoff, segslot, tiles
    assert got == list(off)
    assert val(L, META_MOE, 5) == L.lora_meta_max_tiles(n, S)
    assert [val(L, META_MOE, 10), val(L, META_MOE, 11)] == [n, a["top_k"]]
    assert val(L, MOE, 3) == ws + off[0] and val(L, MOE, 4) == ws + off[4]
    assert val(L, MOE, 8) == ws + B.MOE_CTL_OFFSET                  # the control line in the header
    fused = val(L, MOE, 7)
    assert fused - ws >= off[4] + 4 * 32 * L.lora_meta_max_tiles(n, S)
    assert fused - ws + val(L, MOE, 6) <= need
    # pairs in several metadata chunks: the build's counters sit in the header,
    # its other arrays between the pair metadata and the fused part
    b = moe_args(T=512)
    nb, Sb = b["T"] * b["top_k"], b["E"] * b["L"]
    needb = L.moe_lora_workspace_bytes(b["T"], b["top_k"], b["E"], b["L"], b["R"], b["H"])
    L.raw.stub_reset()
    assert L.moe_lora_gemm1_delta(0x1000, b["H"], b["T"], b["H"], 0x2000, b["R"] * b["H"], 0x3000,
                                  b["I"] * b["R"], 0, 0x4000, b["top_k"], 0x5000, b["E"], b["L"], b["R"], b["I"],
                                  1.0, 0x6000, ws, needb, None) == OK
    wsm = [val(L, META_MOE, i) for i in range(6, 10)]             # ctl, rows, keys, offlen
    assert L.lora_meta_workspace_bytes(nb, Sb) > 0
    assert wsm[0] == ws + 64
    assert min(wsm[1:]) >= val(L, META_MOE, 4) + 4 * 32 * L.lora_meta_max_tiles(nb, Sb)
    assert max(wsm[1:]) < val(L, MOE, 7)
    # w2 reusing gemm1's routing: no metadata launch, the same pair metadata
    need2 = L.moe_lora_w2_workspace_bytes(a["T"], a["top_k"], a["E"], a["L"], a["R"], a["I"])
    L.raw.stub_reset()
    assert L.moe_lora_w2_delta(0x1000, a["I"], a["T"], a["I"], 0x2000, a["R"] * a["I"], 0x3000, a["H"] * a["R"],
                               0x4000, a["top_k"], 0x5000, None, a["E"], a["L"], a["R"], a["H"], 1.0, 0x6000,
                               a["H"], 1, ws, max(need, need2), None) == OK
    assert calls(L) == [0, 0, 0, 0, 0, 0, 0, 1, 0]
    assert val(L, MOE_W2, 3) == ws + off[0] and val(L, MOE_W2, 4) == ws + off[4]
    assert val(L, MOE_W2, 8) == ws + B.MOE_CTL_OFFSET
    assert val(L, MOE_W2, 7) - ws + val(L, MOE_W2, 6) <= max(need, need2)
    # and without the reuse flag it builds the routing itself
    L.raw.stub_reset()
    assert L.moe_lora_w2_delta(0x1000, a["I"], a["T"], a["I"], 0x2000, a["R"] * a["I"], 0x3000, a["H"] * a["R"],
                               0x4000, a["top_k"], 0x5000, 0x7000, a["E"], a["L"], a["R"], a["H"], 1.0, 0x6000,
                               a["H"], 0, ws, need2, None) == OK
    assert calls(L) == [0, 1, 0, 0, 0, 0, 0, 1, 0]


def test_shrink_and_expand_pass_the_tile_bound(L):
    m = meta(0x100000)
    assert L.lora_shrink(0x1000, 256, 40, 256, 0x2000, 0x3000, 4, 1, 8, m, 0x4000, None) == OK
    assert calls(L)[SHRINK] == 1 and val(L, SHRINK, 4) == L.lora_meta_max_tiles(40, 4)
    ss = (ctypes.c_int32 * 2)(256, 128)
    assert L.lora_expand(0x4000, 0x2000, 4, 2, ss, 8, 40, m, 0x3000, 384, 0, 1, None) == OK
    assert calls(L)[EXPAND] == 1 and val(L, EXPAND, 1) == 384 and val(L, EXPAND, 6) == 1


def test_build_call_launches_once_for_decode_batches(L):
    m = meta(0x100000)
    ss = (ctypes.c_int32 * 3)(4096, 1024, 1024)
    need = L.lora_fused_workspace_bytes(256, 32, 3, 16, 4096) + L.lora_meta_workspace_bytes(256, 32)

    def call(n, S, ws_bytes=None):
        nb = ws_bytes if ws_bytes is not None else (L.lora_fused_workspace_bytes(n, S, 3, 16, 4096) +
                                                   L.lora_meta_workspace_bytes(n, S))
        return L.lora_delta_fused_build(0x1000, 4096, n, 4096, 0x2000, 0x3000, 0x4000, S, 3, ss, 16, 0x8000, m,
                                        0x5000, 6144, 0, 0x9000, nb, None)
    assert call(256, 32, need - 1) == EWS
    assert calls(L) == [0] * 9
    assert call(256, 32) == OK
    assert calls(L) == [0, 0, 0, 0, 0, 1, 0, 0, 0]          # the fused launch alone
    assert val(L, FUSED, 9) == 0x8000                        # ... given the slot array
    assert val(L, FUSED, 10) == 0x100000 + 0x40000           # ... and the metadata to write
    assert val(L, FUSED, 11) == L.lora_meta_max_tiles(256, 32)
    for n, S in ((300, 32), (256, 65), (3000, 8)):         # past the one-launch limits: two launches
        L.raw.stub_reset()
        assert call(n, S) == OK, (n, S)
        assert calls(L) == [1, 0, 0, 0, 0, 1, 0, 0, 0], (n, S)
        assert val(L, FUSED, 9) == 0                         # the fused kernel reads the built records
        assert val(L, FUSED, 3) == 0x100000 + 0x40000
        ws_meta = [val(L, META_DENSE, i) for i in range(6, 10)]   # ctl, rows, keys, offlen
        fused_need = L.lora_fused_workspace_bytes(n, S, 3, 16, 4096)
        if L.lora_meta_workspace_bytes(n, S):                # carved after the fused part ...
            assert min(ws_meta[1:]) >= 0x9000 + fused_need
            assert ws_meta[0] == 0x9000 + 64                 # ... its counters in the fixed header
    L.raw.stub_reset()
    assert L.lora_delta_fused_build(0x1000, 4096, 8, 4096, 0x2000, 0x3000, 0x4000, 32, 3, ss, 16, None, m,
                                    0x5000, 6144, 0, 0x9000, need, None) == EINVAL   # no slot array
    assert calls(L) == [0] * 9
