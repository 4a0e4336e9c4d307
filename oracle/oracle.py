"""Python marshalling for the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by the package smoke check and
by the benchmark's CPU-baseline leg; never by the library's product path.
Nothing here does arithmetic of the method: it builds the C file, converts
numpy arrays to pointers and returns numpy results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    L = ctypes.CDLL(path)
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_meta_build.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32,
                                    _i32p, _i32p, _i32p, _i32p]
    L.oracle_moe_keys.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                  ctypes.c_int32, ctypes.c_int32, _i32p]
    L.oracle_shrink_rows.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int32, _u16p, _f32p,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     _i32p, _i32p, ctypes.c_int32, _f64p]
    L.oracle_expand_rows.argtypes = [_f64p, _u16p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                     ctypes.c_int32, _i32p, _i32p, ctypes.c_int32, _u16p,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _f64p]
    L.oracle_moe_gemm1_pairs.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int32,
                                         _i64p, ctypes.c_int64, _i64p, ctypes.c_int64,
                                         ctypes.c_int32, _i32p, ctypes.c_int32, _i32p,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_double, _i32p,
                                         ctypes.c_int32, _f64p]
    L.oracle_expert_workitems.restype = ctypes.c_int32
    L.oracle_expert_workitems.argtypes = [_u32p, ctypes.c_int32, _u16p, ctypes.c_int32, _i32p,
                                          _u32p, _u32p]
    L.oracle_moe_w2_pairs.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int32, _i64p, ctypes.c_int64,
                                      _i64p, ctypes.c_int64, _i32p, ctypes.c_int32, _i32p, _f32p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_double, _u16p, ctypes.c_int64, _i32p, ctypes.c_int32,
                                      _f64p]
    return L


_lib = None
_override = []      # a stack of libraries that replace the default one (tests only)


def lib():
    global _lib
    if _override:
        return _override[-1]
    if _lib is None:
        build(force=False)
        _lib = _bind(_LIB)
    return _lib


class using:
    """Context manager: route every call in this module to another compiled
    copy of the oracle (used by the tests that check the pins catch planted
    mistakes)."""

    def __init__(self, path: str):
        self.L = _bind(path)

    def __enter__(self):
        _override.append(self.L)
        return self

    def __exit__(self, *exc):
        _override.pop()
        return False


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def _p(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- metadata
def meta_build(slot: np.ndarray, num_slots: int):
    """Returns (sorted_rows[n_active], seg_offsets[n_seg+1], seg_slot[n_seg], counts[4])."""
    slot = _c(slot, np.int32)
    n = slot.size
    cap = max(1, min(n, num_slots))
    sorted_rows = np.full(max(n, 1), -7, dtype=np.int32)
    seg_offsets = np.full(cap + 1, -7, dtype=np.int32)
    seg_slot = np.full(cap, -7, dtype=np.int32)
    counts = np.zeros(4, dtype=np.int32)
    lib().oracle_meta_build(_p(slot, _i32p), n, num_slots, _p(sorted_rows, _i32p),
                            _p(seg_offsets, _i32p), _p(seg_slot, _i32p), _p(counts, _i32p))
    na, ns = int(counts[0]), int(counts[1])
    return sorted_rows[:na].copy(), seg_offsets[:ns + 1].copy(), seg_slot[:ns].copy(), counts


def moe_keys(topk_ids: np.ndarray, lora_ids: np.ndarray, num_experts: int, num_loras: int):
    topk_ids = _c(topk_ids, np.int32)
    lora_ids = _c(lora_ids, np.int32)
    T, top_k = topk_ids.shape
    key = np.empty(T * top_k, dtype=np.int32)
    lib().oracle_moe_keys(_p(topk_ids, _i32p), T, top_k, _p(lora_ids, _i32p),
                          num_experts, num_loras, _p(key, _i32p))
    return key


# ---------------------------------------------------------------- dense delta
def shrink_rows(x, k_in, a_pool, scale, num_slots, num_slices, max_rank, slot, rows):
    """xa for the listed rows, [len(rows), num_slices, max_rank] float64.
    Rows without an active slot come back as NaN (the oracle leaves them unwritten)."""
    x = _c(x, np.uint16)
    a_pool, scale, slot = _c(a_pool, np.uint16), _c(scale, np.float32), _c(slot, np.int32)
    rows = _c(rows, np.int32)
    out = np.full((rows.size, num_slices, max_rank), np.nan, dtype=np.float64)
    ldx = x.shape[1] if x.ndim == 2 else k_in
    lib().oracle_shrink_rows(_p(x, _u16p), ldx, k_in, _p(a_pool, _u16p), _p(scale, _f32p),
                             num_slots, num_slices, max_rank, _p(slot, _i32p),
                             _p(rows, _i32p), rows.size, _p(out, _f64p))
    return out


def expand_rows(xa_rows, b_pool, num_slots, slice_sizes, max_rank, slot, rows, y_in,
                offset_start=0, add_inputs=True):
    """y rows after the expand, [len(rows), ldy] float64.  `xa_rows` is
    [len(rows), num_slices, max_rank] (any float dtype, widened exactly)."""
    xa_rows = _c(xa_rows, np.float64)
    b_pool, slot, rows = _c(b_pool, np.uint16), _c(slot, np.int32), _c(rows, np.int32)
    y_in = _c(y_in, np.uint16)
    ss = _c(slice_sizes, np.int32)
    ldy = y_in.shape[1]
    assert offset_start + int(ss.sum()) <= ldy
    out = np.empty((rows.size, ldy), dtype=np.float64)
    lib().oracle_expand_rows(_p(xa_rows, _f64p), _p(b_pool, _u16p), num_slots, ss.size,
                             _p(ss, _i32p), max_rank, _p(slot, _i32p), _p(rows, _i32p),
                             rows.size, _p(y_in, _u16p), ldy, offset_start,
                             1 if add_inputs else 0, _p(out, _f64p))
    return out


def fused_rows(x, k_in, a_pool, b_pool, scale, num_slots, slice_sizes, max_rank, slot, rows,
               y_in, offset_start=0):
    """O-fused: O-expand(O-shrink) with add_inputs = 1, at the listed rows."""
    xa = shrink_rows(x, k_in, a_pool, scale, num_slots, len(slice_sizes), max_rank, slot, rows)
    xa = np.nan_to_num(xa, nan=0.0)   # unwritten rows are never read by the expand
    return expand_rows(xa, b_pool, num_slots, slice_sizes, max_rank, slot, rows, y_in,
                       offset_start, True)


def case_fused_rows(case, rows, offset_start=0, y_in=None):
    return fused_rows(case.x, case.k_in, case.a_pool, case.b_pool, case.scale, case.num_slots,
                      case.slice_sizes, case.max_rank, case.slot, rows,
                      case.y if y_in is None else y_in, offset_start)


# ---------------------------------------------------------------- MoE
def moe_gemm1_pairs(x, w_ptr_a, lora_stride_a, w_ptr_b, lora_stride_b, shared_a, topk_ids,
                    lora_ids, num_experts, num_loras, rank, inter, scale, pairs):
    """out rows for the listed pairs, [len(pairs), 2*inter] float64.  The
    w_ptr tables hold HOST addresses of the bf16 banks (numpy arrays that the
    caller keeps alive)."""
    assert rank <= 256
    x = _c(x, np.uint16)
    T, H = x.shape
    w_ptr_a, w_ptr_b = _c(w_ptr_a, np.int64), _c(w_ptr_b, np.int64)
    topk_ids, lora_ids = _c(topk_ids, np.int32), _c(lora_ids, np.int32)
    pairs = _c(pairs, np.int32)
    out = np.empty((pairs.size, 2 * inter), dtype=np.float64)
    lib().oracle_moe_gemm1_pairs(_p(x, _u16p), H, H, _p(w_ptr_a, _i64p), lora_stride_a,
                                 _p(w_ptr_b, _i64p), lora_stride_b, 1 if shared_a else 0,
                                 _p(topk_ids, _i32p), topk_ids.shape[1], _p(lora_ids, _i32p),
                                 num_experts, num_loras, rank, inter, float(scale),
                                 _p(pairs, _i32p), pairs.size, _p(out, _f64p))
    return out


def host_tables(case, shared_a: bool):
    """Host pointer tables and element strides over a MoeCase's banks, laid out
    like the FlashInfer w_ptr tables: [2, E] (gate, up) or [E]."""
    E, L, R, H, I = case.E, case.L, case.R, case.H, case.I
    if shared_a:
        A, B = case.a_shared, case.b_fused
        ta = np.array([A.ctypes.data + e * L * R * H * 2 for e in range(E)], dtype=np.int64)
        tb = np.array([B.ctypes.data + e * L * 2 * I * R * 2 for e in range(E)], dtype=np.int64)
        return ta, R * H, tb, 2 * I * R
    ta = np.array([[M.ctypes.data + e * L * R * H * 2 for e in range(E)]
                   for M in (case.a_gate, case.a_up)], dtype=np.int64).reshape(-1)
    tb = np.array([[M.ctypes.data + e * L * I * R * 2 for e in range(E)]
                   for M in (case.b_gate, case.b_up)], dtype=np.int64).reshape(-1)
    return ta, R * H, tb, I * R


def case_moe_pairs(case, shared_a: bool, pairs):
    ta, sa, tb, sb = host_tables(case, shared_a)
    return moe_gemm1_pairs(case.x, ta, sa, tb, sb, shared_a, case.topk_ids, case.lora_ids,
                           case.E, case.L, case.R, case.I, case.scale, pairs)


# ---------------------------------------------------------------- MoE w2 (down)
def moe_w2_pairs(x2, w_ptr_a, lora_stride_a, w_ptr_b, lora_stride_b, topk_ids, lora_ids,
                 topk_weights, num_experts, num_loras, rank, H, scale, y, pairs):
    """y rows after the w2 delta for the listed pairs, [len(pairs), H] float64.
    topk_weights may be None (no routing weight).  The w_ptr tables ([E]) hold
    HOST addresses of the bf16 banks, which the caller keeps alive."""
    assert rank <= 256
    x2 = _c(x2, np.uint16)
    I = x2.shape[1]
    y = _c(y, np.uint16)
    w_ptr_a, w_ptr_b = _c(w_ptr_a, np.int64), _c(w_ptr_b, np.int64)
    topk_ids, lora_ids = _c(topk_ids, np.int32), _c(lora_ids, np.int32)
    wts = None if topk_weights is None else _c(topk_weights, np.float32)
    pairs = _c(pairs, np.int32)
    out = np.empty((pairs.size, H), dtype=np.float64)
    lib().oracle_moe_w2_pairs(_p(x2, _u16p), I, I, _p(w_ptr_a, _i64p), lora_stride_a,
                              _p(w_ptr_b, _i64p), lora_stride_b, _p(topk_ids, _i32p),
                              topk_ids.shape[1], _p(lora_ids, _i32p),
                              None if wts is None else _p(wts, _f32p), num_experts, num_loras,
                              rank, H, float(scale), _p(y, _u16p), y.shape[1], _p(pairs, _i32p),
                              pairs.size, _p(out, _f64p))
    return out


def host_tables_w2(case):
    """Host pointer tables ([E]) and element strides over a MoeW2Case's banks."""
    E, L, R, H, I = case.E, case.L, case.R, case.H, case.I
    ta = np.array([case.a_down.ctypes.data + e * L * R * I * 2 for e in range(E)], dtype=np.int64)
    tb = np.array([case.b_down.ctypes.data + e * L * H * R * 2 for e in range(E)], dtype=np.int64)
    return ta, R * I, tb, H * R


def case_moe_w2_pairs(case, pairs, weighted: bool = True, y=None):
    ta, sa, tb, sb = host_tables_w2(case)
    return moe_w2_pairs(case.x2, ta, sa, tb, sb, case.topk_ids, case.lora_ids,
                        case.topk_weights if weighted else None, case.E, case.L, case.R, case.H,
                        case.scale, case.y if y is None else y, pairs)


# ---------------------------------------------------------------- expert-sorted fold
def expert_workitems(expert_offsets, adapted):
    """O-expert-work: [(expert, row_off, rows)] in the order of `adapted`."""
    off = _c(expert_offsets, np.uint32).reshape(-1)
    ad = _c(adapted, np.uint16).reshape(-1)
    cap = max(1, ad.size)
    ie = np.zeros(cap, np.int32)
    io = np.zeros(cap, np.uint32)
    ir = np.zeros(cap, np.uint32)
    offp = _p(off, _u32p) if off.size else None
    adp = _p(ad, _u16p) if ad.size else None
    k = lib().oracle_expert_workitems(offp, off.size, adp, ad.size, _p(ie, _i32p), _p(io, _u32p),
                                      _p(ir, _u32p))
    return [(int(ie[i]), int(io[i]), int(ir[i])) for i in range(k)]


def fold_sorted(x, k_in, base_out, items, pair_slot, a_pool, b_pool, scale, num_slots,
                slice_sizes, max_rank, max_rows=None):
    """The expert-sorted fold (apply_expert_lora_sorted): for each work item
    (e, row_off, rows) whose expert has a pair (pair_slot[e] in [0, num_slots)),
    the pair's delta on rows row_off .. row_off + rows, taken in chunks of at
    most max_rows rows (fold_chunked); other rows keep base_out.  Returns all
    rows, float64.  Items must not overlap."""
    base_out = _c(base_out, np.uint16)
    out = (base_out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    seen = np.zeros(base_out.shape[0], bool)
    for e, r0, nr in items:
        s = int(pair_slot[e])
        if s < 0 or s >= num_slots:
            continue
        step = max(1, nr if max_rows is None else max_rows)
        for c0 in range(r0, r0 + nr, step):
            rows = np.arange(c0, min(r0 + nr, c0 + step), dtype=np.int32)
            assert not seen[rows].any(), "work items overlap"
            seen[rows] = True
            slot = np.full(base_out.shape[0], -1, np.int32)
            slot[rows] = s
            out[rows] = fused_rows(x, k_in, a_pool, b_pool, scale, num_slots, slice_sizes, max_rank,
                                   slot, rows, base_out)
    return out
