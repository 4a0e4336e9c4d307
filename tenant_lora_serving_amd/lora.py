"""Python binding of liblora.so (the C ABI in include/lora.h).

Argument marshalling only: every function checks dtypes, devices and
contiguity, passes raw device pointers, sizes and the current HIP stream to
the library, and raises LoraError on a non-zero status.  Every step of the
path runs in the library's kernels; there is no fallback.  torch provides the
device memory and the stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblora.so")

TILE_ROWS = 16
TILE_WORDS = 32
FUSED_CTL_OFFSET = 0      # byte offset of the control line in a lora_delta_fused workspace
MOE_CTL_OFFSET = 128      # ... in a moe_lora_gemm1_delta / moe_lora_w2_delta workspace

_c_i32, _c_i64, _c_sz, _c_p, _c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_float)


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class _MetaStruct(ctypes.Structure):
    _fields_ = [("sorted_rows", _c_p), ("seg_offsets", _c_p), ("seg_slot", _c_p),
                ("counts", _c_p), ("tiles", _c_p)]


_lib = None


def lib():
    """Load liblora.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tenant_lora_serving_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.lora_meta_max_tiles.restype = _c_i32
        L.lora_meta_max_tiles.argtypes = [_c_i32, _c_i32]
        L.lora_meta_workspace_bytes.restype = _c_sz
        L.lora_meta_workspace_bytes.argtypes = [_c_i32, _c_i32]
        L.lora_meta_build.restype = ctypes.c_int
        L.lora_meta_build.argtypes = [_c_p, _c_i32, _c_i32, _MetaStruct, _c_p, _c_sz, _c_p]
        L.lora_meta_from_offsets.restype = ctypes.c_int
        L.lora_meta_from_offsets.argtypes = [_c_p, _c_i32, _c_p, _c_i32, _c_i32, _MetaStruct, _c_p, _c_sz,
                                             _c_p]
        L.lora_shrink.restype = ctypes.c_int
        L.lora_shrink.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                  _MetaStruct, _c_p, _c_p]
        L.lora_expand.restype = ctypes.c_int
        L.lora_expand.argtypes = [_c_p, _c_p, _c_i32, _c_i32, _c_p, _c_i32, _c_i32, _MetaStruct,
                                  _c_p, _c_i64, _c_i32, _c_i32, _c_p]
        L.lora_fused_workspace_bytes.restype = _c_sz
        L.lora_fused_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]
        L.lora_delta_fused.restype = ctypes.c_int
        L.lora_delta_fused.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                       _c_p, _c_i32, _MetaStruct, _c_p, _c_i64, _c_i32, _c_p, _c_sz,
                                       _c_p]
        L.lora_delta_fused_noalloc.restype = ctypes.c_int
        L.lora_delta_fused_noalloc.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_i32,
                                               _c_i32, _c_p, _c_i32, _MetaStruct, _c_p, _c_i64, _c_i32,
                                               _c_p]
        L.lora_delta_fused_build.restype = ctypes.c_int
        L.lora_delta_fused_build.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                             _c_p, _c_i32, _c_p, _MetaStruct, _c_p, _c_i64, _c_i32, _c_p,
                                             _c_sz, _c_p]
        L.moe_lora_workspace_bytes.restype = _c_sz
        L.moe_lora_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]
        L.moe_lora_gemm1_delta.restype = ctypes.c_int
        L.moe_lora_gemm1_delta.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_i64,
                                           _c_i32, _c_p, _c_i32, _c_p, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_f, _c_p, _c_p, _c_sz, _c_p]
        L.moe_lora_w2_workspace_bytes.restype = _c_sz
        L.moe_lora_w2_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]
        L.moe_lora_w2_delta.restype = ctypes.c_int
        L.moe_lora_w2_delta.argtypes = [_c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_i64, _c_p, _c_i64,
                                        _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _c_f, _c_p, _c_i64, _c_i32, _c_p, _c_sz, _c_p]
        L.moe_lora_meta_layout.restype = ctypes.c_int
        L.moe_lora_meta_layout.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_sz)]
        L.lora_mfma_min_rows.restype = _c_i32
        L.lora_mfma_min_rows.argtypes = []
        L.lora_set_mfma_min_rows.restype = None
        L.lora_set_mfma_min_rows.argtypes = [_c_i32]
        L.lora_status_string.restype = ctypes.c_char_p
        L.lora_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


EXPORTED = ["lora_meta_max_tiles", "lora_meta_workspace_bytes", "lora_meta_build",
            "lora_meta_from_offsets", "lora_shrink",
            "lora_expand", "lora_fused_workspace_bytes", "lora_delta_fused", "lora_delta_fused_noalloc",
            "lora_delta_fused_build",
            "moe_lora_workspace_bytes", "moe_lora_gemm1_delta", "moe_lora_w2_workspace_bytes",
            "moe_lora_w2_delta", "moe_lora_meta_layout", "lora_mfma_min_rows",
            "lora_set_mfma_min_rows", "lora_status_string"]


def _check(fn: str, status: int):
    if status != 0:
        raise LoraError(fn, status, lib().lora_status_string(status).decode())


@dataclass
class WsStatus:
    """A fused or MoE workspace's control line."""
    error: int       # 1 once a bounded wait gave up (never cleared by the library)
    calls: int       # calls completed on the workspace (low 31 bits of the last tag)
    running: int     # tiles counted by an unfinished call: 0 between calls

    @property
    def ok(self) -> bool:
        return self.error == 0 and self.running == 0


def ws_status(ws: torch.Tensor, moe: bool = False) -> WsStatus:
    """Read a workspace's control line (synchronizes with the device)."""
    o = MOE_CTL_OFFSET if moe else FUSED_CTL_OFFSET
    err, tag, run = ws[o:o + 12].view(torch.int32).cpu().tolist()
    return WsStatus(err, tag & 0x7FFFFFFF, run)


def _check_ws(fn: str, ws: torch.Tensor, moe: bool, stream):
    (stream or torch.cuda.current_stream()).synchronize()
    st = ws_status(ws, moe)
    if not st.ok:
        raise LoraError(fn, -100, f"workspace control line reports {st}")


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _rows_ld(t: torch.Tensor, name: str):
    """Row-major 2-D bf16 with unit column stride: returns (ptr, leading dim)."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return _dev(t, name, torch.bfloat16, contiguous=False), t.stride(0)


def set_mfma_min_rows(rows: int):
    """Override the MFMA row threshold for the calling thread (rows <= 0: back
    to the default)."""
    lib().lora_set_mfma_min_rows(int(rows))


def mfma_min_rows() -> int:
    return int(lib().lora_mfma_min_rows())


# ---------------------------------------------------------------- metadata
@dataclass
class LoraMeta:
    """Device buffers of one batch's routing metadata (lora_meta_t) and the
    workspace of its build."""
    n: int
    num_slots: int
    sorted_rows: torch.Tensor
    seg_offsets: torch.Tensor
    seg_slot: torch.Tensor
    counts: torch.Tensor
    tiles: torch.Tensor
    ws: torch.Tensor

    @classmethod
    def allocate(cls, n: int, num_slots: int, device="cuda"):
        L = lib()
        cap = min(n, num_slots)
        tb = int(L.lora_meta_max_tiles(n, num_slots))
        wsb = int(L.lora_meta_workspace_bytes(n, num_slots))
        i32 = dict(dtype=torch.int32, device=device)
        return cls(n, num_slots,
                   torch.empty(max(n, 1), **i32), torch.empty(cap + 1, **i32),
                   torch.empty(max(cap, 1), **i32), torch.zeros(8, **i32),
                   torch.empty(max(tb, 1) * TILE_WORDS, **i32),
                   torch.zeros(max(wsb, 16), dtype=torch.uint8, device=device))

    def struct(self) -> _MetaStruct:
        return _MetaStruct(self.sorted_rows.data_ptr(), self.seg_offsets.data_ptr(),
                           self.seg_slot.data_ptr(), self.counts.data_ptr(), self.tiles.data_ptr())


def lora_meta_build(slot: torch.Tensor, num_slots: int, meta: LoraMeta | None = None,
                    stream=None) -> LoraMeta:
    n = slot.numel()
    if meta is None:
        meta = LoraMeta.allocate(n, num_slots, slot.device)
    assert meta.n == n and meta.num_slots == num_slots, "metadata buffers sized for another batch"
    p = _dev(slot, "slot", torch.int32)
    st = lib().lora_meta_build(p, n, num_slots, meta.struct(), meta.ws.data_ptr(), meta.ws.numel(),
                               _stream(stream))
    _check("lora_meta_build", st)
    return meta


# ---------------------------------------------------------------- dense delta
def lora_meta_from_offsets(expert_offsets: torch.Tensor, expert_slot: torch.Tensor, n: int,
                           num_slots: int, meta: LoraMeta | None = None, stream=None) -> LoraMeta:
    """Metadata of the expert-sorted fold: sorted row r takes the pool slot
    expert_slot[e] of the expert e whose block of the expert_offsets prefix
    sum ([E + 1] uint32 as int32 bits) holds it."""
    E = expert_slot.numel()
    if expert_offsets.numel() != E + 1:
        raise ValueError("expert_offsets must have num_experts + 1 entries")
    if expert_offsets.dtype not in (torch.int32, torch.uint32):
        raise TypeError("expert_offsets must be 32-bit")
    if meta is None:
        meta = LoraMeta.allocate(n, num_slots, expert_slot.device)
    assert meta.n == n and meta.num_slots == num_slots, "metadata buffers sized for another batch"
    st = lib().lora_meta_from_offsets(_dev(expert_offsets, "expert_offsets"), E,
                                      _dev(expert_slot, "expert_slot", torch.int32), n, num_slots,
                                      meta.struct(), meta.ws.data_ptr(), meta.ws.numel(), _stream(stream))
    _check("lora_meta_from_offsets", st)
    return meta


def _pool_dims(a_pool=None, b_pool=None):
    if a_pool is not None:
        if a_pool.dim() != 4:
            raise ValueError("a_pool must be [num_slots, num_slices, max_rank, k_in]")
    if b_pool is not None and b_pool.dim() != 3:
        raise ValueError("b_pool must be [num_slots, N, max_rank]")


def lora_shrink(x: torch.Tensor, a_pool: torch.Tensor, scale: torch.Tensor, meta: LoraMeta,
                xa: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """xa[l, i, :] = scale[s] * A_s[l] @ x[i] for active rows (others untouched)."""
    _pool_dims(a_pool=a_pool)
    S, Lsl, R, k_in = a_pool.shape
    xp, ldx = _rows_ld(x, "x")
    n = x.shape[0]
    if x.shape[1] < k_in:
        raise ValueError("x has fewer columns than k_in")
    if xa is None:
        xa = torch.zeros((Lsl, n, R), dtype=torch.float32, device=x.device)
    st = lib().lora_shrink(xp, ldx, n, k_in, _dev(a_pool, "a_pool", torch.bfloat16),
                           _dev(scale, "scale", torch.float32), S, Lsl, R, meta.struct(),
                           _dev(xa, "xa", torch.float32), _stream(stream))
    _check("lora_shrink", st)
    return xa


def lora_expand(xa: torch.Tensor, b_pool: torch.Tensor, slice_sizes, meta: LoraMeta,
                y: torch.Tensor, offset_start: int = 0, add_inputs: bool = True,
                stream=None) -> torch.Tensor:
    """y[i, window] (+)= xa[l, i] @ B_s[slice]^T for active rows, in place."""
    _pool_dims(b_pool=b_pool)
    S, N, R = b_pool.shape
    ss = (ctypes.c_int32 * len(slice_sizes))(*[int(v) for v in slice_sizes])
    if sum(slice_sizes) != N:
        raise ValueError("slice sizes must add up to b_pool's N")
    yp, ldy = _rows_ld(y, "y")
    st = lib().lora_expand(_dev(xa, "xa", torch.float32), _dev(b_pool, "b_pool", torch.bfloat16), S,
                           len(slice_sizes), ss, R, y.shape[0], meta.struct(), yp, ldy,
                           int(offset_start), 1 if add_inputs else 0, _stream(stream))
    _check("lora_expand", st)
    return y


def fused_workspace(n: int, num_slots: int, num_slices: int, max_rank: int, k_in: int,
                    device="cuda") -> torch.Tensor:
    b = int(lib().lora_fused_workspace_bytes(n, num_slots, num_slices, max_rank, k_in))
    return torch.zeros(max(b, 16), dtype=torch.uint8, device=device)


def lora_delta_fused(x: torch.Tensor, a_pool: torch.Tensor, b_pool: torch.Tensor,
                     scale: torch.Tensor, slice_sizes, meta: LoraMeta, y: torch.Tensor,
                     offset_start: int = 0, ws: torch.Tensor | None = None,
                     stream=None, check: bool = False) -> torch.Tensor:
    """y[i, window] += (scale[s] * x[i] @ A_s^T) @ B_s^T for active rows, in place.
    check: synchronize afterwards and raise if the workspace's error word is set."""
    _pool_dims(a_pool, b_pool)
    S, Lsl, R, k_in = a_pool.shape
    if len(slice_sizes) != Lsl or sum(slice_sizes) != b_pool.shape[1]:
        raise ValueError("slice sizes do not match the pools")
    xp, ldx = _rows_ld(x, "x")
    yp, ldy = _rows_ld(y, "y")
    n = x.shape[0]
    if y.shape[0] != n:
        raise ValueError("x and y row counts differ")
    if ws is None:
        ws = fused_workspace(n, S, Lsl, R, k_in, x.device)
    ss = (ctypes.c_int32 * Lsl)(*[int(v) for v in slice_sizes])
    st = lib().lora_delta_fused(xp, ldx, n, k_in, _dev(a_pool, "a_pool", torch.bfloat16),
                                _dev(b_pool, "b_pool", torch.bfloat16),
                                _dev(scale, "scale", torch.float32), S, Lsl, ss, R, meta.struct(),
                                yp, ldy, int(offset_start), _dev(ws, "ws", torch.uint8),
                                ws.numel(), _stream(stream))
    _check("lora_delta_fused", st)
    if check:
        _check_ws("lora_delta_fused", ws, False, stream)
    return y


def fused_build_workspace(n: int, num_slots: int, num_slices: int, max_rank: int, k_in: int,
                          device="cuda") -> torch.Tensor:
    """Workspace of lora_delta_fused_build: the fused workspace, then the
    metadata build's (it also serves lora_delta_fused)."""
    L = lib()
    b = int(L.lora_fused_workspace_bytes(n, num_slots, num_slices, max_rank, k_in))
    b += int(L.lora_meta_workspace_bytes(n, num_slots))
    return torch.zeros(max(b, 16), dtype=torch.uint8, device=device)


def lora_delta_fused_build(x: torch.Tensor, a_pool: torch.Tensor, b_pool: torch.Tensor,
                           scale: torch.Tensor, slice_sizes, slot: torch.Tensor, y: torch.Tensor,
                           meta: LoraMeta | None = None, offset_start: int = 0,
                           ws: torch.Tensor | None = None, stream=None, check: bool = False) -> LoraMeta:
    """lora_meta_build(slot) and lora_delta_fused in one call (one launch for
    decode-sized batches): y is updated in place and the batch's metadata,
    for later calls of the step, is written to meta (returned).
    check: synchronize afterwards and raise if the workspace's error word is set."""
    _pool_dims(a_pool, b_pool)
    S, Lsl, R, k_in = a_pool.shape
    if len(slice_sizes) != Lsl or sum(slice_sizes) != b_pool.shape[1]:
        raise ValueError("slice sizes do not match the pools")
    xp, ldx = _rows_ld(x, "x")
    yp, ldy = _rows_ld(y, "y")
    n = x.shape[0]
    if y.shape[0] != n or slot.numel() != n:
        raise ValueError("x, y and slot row counts differ")
    if meta is None:
        meta = LoraMeta.allocate(n, S, x.device)
    assert meta.n == n and meta.num_slots == S, "metadata buffers sized for another batch"
    if ws is None:
        ws = fused_build_workspace(n, S, Lsl, R, k_in, x.device)
    ss = (ctypes.c_int32 * Lsl)(*[int(v) for v in slice_sizes])
    st = lib().lora_delta_fused_build(xp, ldx, n, k_in, _dev(a_pool, "a_pool", torch.bfloat16),
                                      _dev(b_pool, "b_pool", torch.bfloat16),
                                      _dev(scale, "scale", torch.float32), S, Lsl, ss, R,
                                      _dev(slot, "slot", torch.int32), meta.struct(), yp, ldy,
                                      int(offset_start), _dev(ws, "ws", torch.uint8), ws.numel(),
                                      _stream(stream))
    _check("lora_delta_fused_build", st)
    if check:
        _check_ws("lora_delta_fused_build", ws, False, stream)
    return meta


NOALLOC_SCRATCH_BYTES = 16 << 20   # the fixed device buffer behind lora_delta_fused_noalloc


def lora_delta_fused_noalloc(x: torch.Tensor, a_pool: torch.Tensor, b_pool: torch.Tensor,
                             scale: torch.Tensor, slice_sizes, meta: LoraMeta, y: torch.Tensor,
                             offset_start: int = 0, stream=None) -> torch.Tensor:
    """lora_delta_fused on the library's own fixed device buffer: no workspace
    argument, nothing allocated (for callers that cannot allocate).  Calls
    whose workspace would exceed the buffer raise (status -5)."""
    _pool_dims(a_pool, b_pool)
    S, Lsl, R, k_in = a_pool.shape
    if len(slice_sizes) != Lsl or sum(slice_sizes) != b_pool.shape[1]:
        raise ValueError("slice sizes do not match the pools")
    xp, ldx = _rows_ld(x, "x")
    yp, ldy = _rows_ld(y, "y")
    n = x.shape[0]
    if y.shape[0] != n:
        raise ValueError("x and y row counts differ")
    ss = (ctypes.c_int32 * Lsl)(*[int(v) for v in slice_sizes])
    st = lib().lora_delta_fused_noalloc(xp, ldx, n, k_in, _dev(a_pool, "a_pool", torch.bfloat16),
                                        _dev(b_pool, "b_pool", torch.bfloat16),
                                        _dev(scale, "scale", torch.float32), S, Lsl, ss, R, meta.struct(),
                                        yp, ldy, int(offset_start), _stream(stream))
    _check("lora_delta_fused_noalloc", st)
    return y


# ---------------------------------------------------------------- MoE
def moe_workspace(T: int, top_k: int, num_experts: int, num_loras: int, rank: int, H: int,
                  device="cuda") -> torch.Tensor:
    b = int(lib().moe_lora_workspace_bytes(T, top_k, num_experts, num_loras, rank, H))
    return torch.zeros(max(b, 16), dtype=torch.uint8, device=device)


def moe_lora_gemm1_delta(hidden_states: torch.Tensor, w_ptr_a: torch.Tensor, lora_stride_a: int,
                         w_ptr_b: torch.Tensor, lora_stride_b: int, topk_ids: torch.Tensor,
                         lora_ids: torch.Tensor, rank: int, intermediate_size: int, *,
                         num_loras: int, scale: float = 1.0, out: torch.Tensor | None = None,
                         ws: torch.Tensor | None = None, stream=None,
                         check: bool = False) -> torch.Tensor:
    """[T, top_k, 2I] gate/up delta per routed pair.  A 2-D [2, E] pointer
    table selects the regular form, a 1-D [E] table the shared-A form."""
    shared = w_ptr_a.dim() == 1
    if (w_ptr_b.dim() == 1) != shared:
        raise ValueError("w_ptr_a and w_ptr_b must both be 1-D or both be [2, E]")
    E = w_ptr_a.shape[-1]
    if not shared and w_ptr_a.shape[0] != 2:
        raise ValueError("regular pointer tables are [2, num_experts]")
    T, H = hidden_states.shape
    top_k = topk_ids.shape[1]
    xp, ldx = _rows_ld(hidden_states, "hidden_states")
    if out is None:
        out = torch.empty((T, top_k, 2 * intermediate_size), dtype=torch.bfloat16,
                          device=hidden_states.device)
    if ws is None:
        ws = moe_workspace(T, top_k, E, num_loras, rank, H, hidden_states.device)
    st = lib().moe_lora_gemm1_delta(
        xp, ldx, T, H, _dev(w_ptr_a, "w_ptr_a", torch.int64), int(lora_stride_a),
        _dev(w_ptr_b, "w_ptr_b", torch.int64), int(lora_stride_b), 1 if shared else 0,
        _dev(topk_ids, "topk_ids", torch.int32), top_k, _dev(lora_ids, "lora_ids", torch.int32),
        E, int(num_loras), int(rank), int(intermediate_size), float(scale),
        _dev(out, "out", torch.bfloat16), _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    _check("moe_lora_gemm1_delta", st)
    if check:
        _check_ws("moe_lora_gemm1_delta", ws, True, stream)
    return out


def moe_w2_workspace(T: int, top_k: int, num_experts: int, num_loras: int, rank: int, I: int,
                     device="cuda") -> torch.Tensor:
    b = int(lib().moe_lora_w2_workspace_bytes(T, top_k, num_experts, num_loras, rank, I))
    return torch.zeros(max(b, 16), dtype=torch.uint8, device=device)


def _pair_rows(t: torch.Tensor, name: str, n_pairs: int):
    """[T*top_k, W] or [T, top_k, W] bf16 rows with unit column stride."""
    if t.dim() == 3:
        t = t.view(-1, t.shape[2])
    if t.dim() != 2 or t.shape[0] != n_pairs:
        raise ValueError(f"{name} must hold one row per (token, slot) pair")
    return t


def moe_lora_w2_delta(x2: torch.Tensor, w_ptr_a: torch.Tensor, lora_stride_a: int,
                      w_ptr_b: torch.Tensor, lora_stride_b: int, topk_ids: torch.Tensor,
                      lora_ids: torch.Tensor, rank: int, y: torch.Tensor, *, num_loras: int,
                      topk_weights: torch.Tensor | None = None, scale: float = 1.0,
                      ws: torch.Tensor | None = None, reuse_routing: bool = False,
                      stream=None, check: bool = False) -> torch.Tensor:
    """Add the routed down-projection delta to y ([T*top_k, H] or [T, top_k, H])
    in place; x2 holds the pairs' activated gemm1 outputs, [T*top_k, I].
    reuse_routing: ws holds the pair metadata of this routing from the
    previous MoE call on it (the gemm1 delta), so it is not rebuilt."""
    if reuse_routing and ws is None:
        raise ValueError("reuse_routing needs the workspace of the previous MoE call")
    if w_ptr_a.dim() != 1 or w_ptr_b.dim() != 1:
        raise ValueError("w2 pointer tables are [num_experts]")
    E = w_ptr_a.shape[0]
    T, top_k = topk_ids.shape
    x2v = _pair_rows(x2, "x2", T * top_k)
    yv = _pair_rows(y, "y", T * top_k)
    I, H = x2v.shape[1], yv.shape[1]
    xp, ldx = _rows_ld(x2v, "x2")
    yp, ldy = _rows_ld(yv, "y")
    wp = None
    if topk_weights is not None:
        if topk_weights.shape != (T, top_k):
            raise ValueError("topk_weights must be [T, top_k]")
        wp = _dev(topk_weights, "topk_weights", torch.float32)
    if ws is None:
        ws = moe_w2_workspace(T, top_k, E, num_loras, rank, I, x2.device)
    st = lib().moe_lora_w2_delta(
        xp, ldx, T, I, _dev(w_ptr_a, "w_ptr_a", torch.int64), int(lora_stride_a),
        _dev(w_ptr_b, "w_ptr_b", torch.int64), int(lora_stride_b),
        _dev(topk_ids, "topk_ids", torch.int32), top_k, _dev(lora_ids, "lora_ids", torch.int32), wp,
        E, int(num_loras), int(rank), H, float(scale), yp, ldy, 1 if reuse_routing else 0,
        _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    _check("moe_lora_w2_delta", st)
    if check:
        _check_ws("moe_lora_w2_delta", ws, True, stream)
    return y


def moe_counts(ws: torch.Tensor) -> torch.Tensor:
    """{n_active_pairs, n_segments, n_invalid_pairs, n_long_segments} of the last MoE call."""
    return ws[:16].view(torch.int32)


def moe_meta_view(ws: torch.Tensor, T: int, top_k: int, num_experts: int, num_loras: int) -> LoraMeta:
    """The pair metadata the last MoE call built in ws, as views of ws (for n =
    T * top_k pairs and S = num_loras * num_experts (adapter, expert) keys)."""
    off = (_c_sz * 5)()
    _check("moe_lora_meta_layout", lib().moe_lora_meta_layout(T, top_k, num_experts, num_loras, off))
    n, S = T * top_k, num_experts * num_loras
    cap = min(n, S)
    tb = int(lib().lora_meta_max_tiles(n, S))

    def view(i, count):
        return ws[off[i]:off[i] + 4 * count].view(torch.int32)
    return LoraMeta(n, S, view(1, n), view(2, cap + 1), view(3, cap), view(0, 8),
                    view(4, tb * TILE_WORDS), ws[:0])


def fill_w_ptr(*banks: torch.Tensor):
    """Pointer table and adapter stride over expert-major LoRA banks, the form
    bgmv_moe_gemm1_lora_delta's w_ptr_a / w_ptr_b take.  Each bank is a
    contiguous [num_experts, num_loras, rows, cols] bf16 device tensor; entry
    [s][e] is the address of bank s's block for expert e, and adapter l's
    matrix starts l * stride elements past it, stride = rows * cols.  One bank
    gives the 1-D [num_experts] table (one shared A, or the fused [2I, rank] B),
    two give [2, num_experts] (gate, up).  Returns (table on the banks' device,
    stride).  The banks must outlive every call that uses the table."""
    if not banks or len(banks) > 2:
        raise ValueError("fill_w_ptr takes one bank (shared / fused form) or two (gate, up)")
    shapes = {tuple(b.shape) for b in banks}
    if len(shapes) != 1 or banks[0].dim() != 4:
        raise ValueError("banks must all be [num_experts, num_loras, rows, cols]")
    for i, b in enumerate(banks):
        _dev(b, f"bank {i}", torch.bfloat16)
    E, L, r, c = banks[0].shape
    block = L * r * c * banks[0].element_size()
    tab = [[b.data_ptr() + e * block for e in range(E)] for b in banks]
    t = torch.tensor(tab if len(banks) == 2 else tab[0], dtype=torch.int64)
    return t.to(banks[0].device), r * c


# ---------------------------------------------------------------- expert-sorted and router folds
def apply_expert_lora_sorted(x: torch.Tensor, base_out: torch.Tensor, expert_offsets: torch.Tensor,
                             expert_slot: torch.Tensor, a_pool: torch.Tensor, b_pool: torch.Tensor,
                             scale: torch.Tensor, meta: LoraMeta | None = None,
                             ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fold each adapted expert's pair onto its block of the expert-sorted
    output in place: base_out[r] += delta of pair expert_slot[e] for the rows
    r of expert e (one pool slot per pair, one output slice)."""
    n = x.shape[0]
    meta = lora_meta_from_offsets(expert_offsets, expert_slot, n, a_pool.shape[0], meta, stream)
    return lora_delta_fused(x, a_pool, b_pool, scale, (b_pool.shape[1],), meta, base_out, ws=ws,
                            stream=stream)


def apply_router_lora(router_in: torch.Tensor, gate_logits: torch.Tensor, a: torch.Tensor,
                      b: torch.Tensor, scale: float, meta: LoraMeta | None = None,
                      ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fold the router pair (a [R, hidden], b [num_experts, R]) onto
    gate_logits [n, num_experts] in place: one block of all n rows."""
    n = router_in.shape[0]
    dev = router_in.device
    offsets = torch.tensor([0, n], dtype=torch.int32).to(dev, non_blocking=True)
    slot0 = torch.zeros(1, dtype=torch.int32, device=dev)
    meta = lora_meta_from_offsets(offsets, slot0, n, 1, meta, stream)
    scale_t = torch.full((1,), float(scale), dtype=torch.float32, device=dev)
    return lora_delta_fused(router_in, a.reshape(1, 1, *a.shape), b.reshape(1, *b.shape), scale_t,
                            (b.shape[0],), meta, gate_logits, ws=ws, stream=stream)


# ---------------------------------------------------------------- logits and embedding variants
def add_lora_logits(y: torch.Tensor, x: torch.Tensor, a_pool: torch.Tensor, b_pool: torch.Tensor,
                    scale: torch.Tensor, sampler_slot: torch.Tensor, meta: LoraMeta | None = None,
                    ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """LM-head logits delta: y[i, :vocab] += (scale[s] * x[i] @ A_s^T) @ B_s^T
    for each sampled row i with s = sampler_slot[i] (a_pool [S, 1, R, hidden],
    b_pool [S, vocab, R]), in place."""
    meta = lora_meta_build(sampler_slot, a_pool.shape[0], meta, stream)
    return lora_delta_fused(x, a_pool, b_pool, scale, (b_pool.shape[1],), meta, y, ws=ws,
                            stream=stream)


def add_lora_embedding(y: torch.Tensor, x: torch.Tensor, b_pool: torch.Tensor, slot: torch.Tensor,
                       add_inputs: bool = True, meta: LoraMeta | None = None,
                       stream=None) -> torch.Tensor:
    """Embedding delta, expand only: y[i] (+)= x[i] @ B_s^T for s = slot[i],
    with x [n, R] float32 (the adapter's embedding rows of the tokens) and
    b_pool [S, hidden, R]."""
    if x.dtype != torch.float32 or x.dim() != 2:
        raise TypeError("x must be a 2-D float32 tensor [n, R]")
    meta = lora_meta_build(slot, b_pool.shape[0], meta, stream)
    return lora_expand(x.reshape(1, *x.shape), b_pool, (b_pool.shape[1],), meta, y,
                       add_inputs=add_inputs, stream=stream)
