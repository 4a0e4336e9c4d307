"""Seeded synthetic inputs for the routed LoRA delta workloads.

This module only draws random numbers and lays them out in the pool layouts the
library and the oracle both take.  It holds none of the delta's arithmetic: no
shrink, no expand, no sort.  Both the HIP path (through the binding) and the
CPU oracle (through the tests) are fed from here, and from nowhere else.

Layouts (the metrale `lora_delta` page, `LoraPair` and `LoraRoute`):
  x       [n, k_in]                 bf16 bit patterns (uint16), row-major
  a_pool  [S, n_slices, R, k_in]    bf16, rows r >= rank_s are zero
  b_pool  [S, N, R]                 bf16, N = sum(slice_sizes), cols r >= rank_s zero
  scale   [S]                       float32
  y       [n, N]                    bf16
MoE banks (the FlashInfer `bgmv_moe_gemm1_lora_delta` page, `w_ptr_a/w_ptr_b`):
  A bank  [E, L, R, H]   B bank [E, L, I or 2I, R]   (adapter stride R*H, I*R, 2I*R)

Every draw comes from numpy's PCG64 generator seeded by the caller, in a fixed
order: routing, ranks, A, B, x, y.  Values are drawn in float32 and rounded to
bf16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


# ---------------------------------------------------------------- bf16 coding
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat_in = a.reshape(-1).view(np.uint32)
    out = np.empty(flat_in.shape, dtype=np.uint16)
    step = 1 << 20                       # cache-sized chunks
    tmp = np.empty(min(step, flat_in.size), dtype=np.uint32)
    for lo in range(0, flat_in.size, step):
        u = flat_in[lo:lo + step]
        t = tmp[:u.size]
        np.right_shift(u, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        np.add(t, np.uint32(0x7FFF), out=t)
        np.add(t, u, out=t)
        np.right_shift(t, 16, out=t)
        out[lo:lo + step] = t
    nan = np.isnan(a.reshape(-1))
    if nan.any():
        out[nan] = 0x7FC0
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


# ---------------------------------------------------------------- dense case
@dataclass
class DenseCase:
    name: str
    n: int
    k_in: int
    slice_sizes: tuple
    num_slots: int
    max_rank: int
    ranks: np.ndarray          # [S] int32, true rank of each slot
    slot: np.ndarray           # [n] int32, negative = no delta
    scale: np.ndarray          # [S] float32
    x: np.ndarray              # [n, k_in] uint16
    a_pool: np.ndarray         # [S, L, R, k_in] uint16
    b_pool: np.ndarray         # [S, N, R] uint16
    y: np.ndarray              # [n, N] uint16
    meta: dict = field(default_factory=dict)

    @property
    def num_slices(self) -> int:
        return len(self.slice_sizes)

    @property
    def n_out(self) -> int:
        return int(sum(self.slice_sizes))


def _pools(rng, num_slots, num_slices, max_rank, k_in, n_out, ranks):
    """A rows < rank_s ~ N(0, 1/k_in); B cols < rank_s ~ N(0, 1/rank_s); rest zero."""
    if np.all(ranks == max_rank):
        a_pool = _normal_bf16(rng, (num_slots, num_slices, max_rank, k_in), 1.0 / np.sqrt(k_in))
        b_pool = _normal_bf16(rng, (num_slots, n_out, max_rank), 1.0 / np.sqrt(max_rank))
        return a_pool, b_pool
    a_pool = np.zeros((num_slots, num_slices, max_rank, k_in), dtype=np.uint16)
    for s in range(num_slots):
        r = int(ranks[s])
        a_pool[s, :, :r, :] = _normal_bf16(rng, (num_slices, r, k_in), 1.0 / np.sqrt(k_in))
    b_pool = np.zeros((num_slots, n_out, max_rank), dtype=np.uint16)
    for s in range(num_slots):
        r = int(ranks[s])
        b_pool[s, :, :r] = _normal_bf16(rng, (n_out, r), 1.0 / np.sqrt(r))
    return a_pool, b_pool


def make_dense(seed, *, n: int, k_in: int, slice_sizes, num_slots: int,
               max_rank: int, ranks=None, rank_choices=None, slot=None,
               slot_kind: str = "uniform_neg", scale_num: float = 16.0,
               scale_fixed: float | None = None, neg_frac: float = 0.0,
               name: str = "custom") -> DenseCase:
    """Generic dense workload.  `slot_kind`:
      uniform_neg  slot uniform over {-1, 0, ..., S-1}
      uniform      slot uniform over {0, ..., S-1}
      zipf         P(slot = k-1) proportional to 1/k, k = 1..S
      perm         a random permutation of 0..n-1 (needs n == S)
    after which each row becomes -1 with probability `neg_frac`.
    scale_s = scale_num / rank_s unless `scale_fixed` is given.  `seed` is an
    int or an already-seeded numpy Generator (drawn from in place)."""
    rng = np.random.default_rng(seed)
    slice_sizes = tuple(int(v) for v in slice_sizes)
    n_out = sum(slice_sizes)
    # routing
    if slot is None:
        if slot_kind == "uniform_neg":
            slot = rng.integers(-1, num_slots, size=n)
        elif slot_kind == "uniform":
            slot = rng.integers(0, num_slots, size=n)
        elif slot_kind == "zipf":
            p = 1.0 / np.arange(1, num_slots + 1, dtype=np.float64)
            p /= p.sum()
            slot = rng.choice(num_slots, size=n, p=p)
        elif slot_kind == "perm":
            assert n == num_slots
            slot = rng.permutation(num_slots)
        else:
            raise ValueError(slot_kind)
        slot = np.asarray(slot, dtype=np.int64)
        if neg_frac > 0:
            slot = np.where(rng.random(n) < neg_frac, -1, slot)
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    # ranks
    if ranks is None:
        if rank_choices is None:
            ranks = np.full(num_slots, max_rank)
        else:
            ranks = rng.choice(np.asarray(rank_choices), size=num_slots)
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    assert ranks.max(initial=0) <= max_rank
    a_pool, b_pool = _pools(rng, num_slots, len(slice_sizes), max_rank, k_in, n_out, ranks)
    x = _normal_bf16(rng, (n, k_in), 1.0)
    y = _normal_bf16(rng, (n, n_out), 1.0)
    if scale_fixed is not None:
        scale = np.full(num_slots, scale_fixed, dtype=np.float32)
    else:
        scale = (np.float32(scale_num) / np.maximum(ranks, 1).astype(np.float32)).astype(np.float32)
    return DenseCase(name, n, k_in, slice_sizes, num_slots, max_rank, ranks, slot,
                     scale, x, a_pool, b_pool, y)


# ---------------------------------------------------------------- the five workloads
def tiny_bgmv(seed: int = 1) -> DenseCase:
    """8 rows, k_in = n_out = 256, 4 slots of true ranks {4,8,8,2} padded to 8,
    scale 16/r, slot uniform over {-1,0,1,2,3}."""
    return make_dense(seed, n=8, k_in=256, slice_sizes=(256,), num_slots=4, max_rank=8,
                      ranks=[4, 8, 8, 2], slot_kind="uniform_neg", scale_num=16.0,
                      name="tiny routed BGMV n=8 k=256 N=256 R=8")


def decode_bgmv(seed: int = 2, n: int = 256) -> DenseCase:
    """Decode BGMV at the Llama-3-8B QKV shape: 256 one-token rows, k_in 4096,
    slices (4096, 1024, 1024), 32 adapters at max rank 16 with true ranks in
    {8, 16}, Zipf(1) routing with 5% of rows unadapted, scale 32/r."""
    return make_dense(seed, n=n, k_in=4096, slice_sizes=(4096, 1024, 1024), num_slots=32,
                      max_rank=16, rank_choices=[8, 16], slot_kind="zipf", neg_frac=0.05,
                      scale_num=32.0, name="decode BGMV llama3-8b qkv n=256 S=32 R=16")


def prefill_sgmv(seed: int = 3, n_seq: int = 16, len_lo: int = 64, len_hi: int = 1024,
                 k_in: int = 4096, slice_sizes=(14336, 14336)) -> DenseCase:
    """Prefill SGMV: 16 sequences of lengths uniform in [64, 1024], rows of a
    sequence contiguous with one adapter drawn uniformly from 16; k_in 4096,
    gate_up slices (14336, 14336), rank 64, scale 2."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi + 1, size=n_seq)
    seq_slot = rng.integers(0, 16, size=n_seq)
    slot = np.repeat(seq_slot, lens).astype(np.int32)
    # the rest of the case keeps drawing from the same stream
    c = make_dense(rng, n=int(lens.sum()), k_in=k_in, slice_sizes=slice_sizes,
                   num_slots=16, max_rank=64, ranks=np.full(16, 64), slot=slot,
                   scale_fixed=2.0, name="prefill SGMV 16 seqs k=4096 N=2x14336 R=64")
    c.meta["seq_lens"] = lens
    c.meta["seq_slot"] = seq_slot
    return c


def no_reuse(seed: int = 4) -> DenseCase:
    """Worst case without reuse: 1024 rows, each with its own adapter of a
    1024-slot pool, k_in = n_out = 4096, rank 32, slot a random permutation."""
    return make_dense(seed, n=1024, k_in=4096, slice_sizes=(4096,), num_slots=1024,
                      max_rank=32, ranks=np.full(1024, 32), slot_kind="perm",
                      scale_fixed=1.0, name="no-reuse n=1024 S=1024 k=4096 N=4096 R=32")


# ---------------------------------------------------------------- MoE case
@dataclass
class MoeCase:
    name: str
    T: int
    H: int
    E: int
    top_k: int
    I: int
    R: int
    L: int
    scale: float
    topk_ids: np.ndarray      # [T, top_k] int32
    lora_ids: np.ndarray      # [T] int32, -1 = none
    x: np.ndarray             # [T, H] uint16
    a_gate: np.ndarray        # [E, L, R, H]
    a_up: np.ndarray          # [E, L, R, H]
    b_gate: np.ndarray        # [E, L, I, R]
    b_up: np.ndarray          # [E, L, I, R]
    a_shared: np.ndarray      # [E, L, R, H]
    b_fused: np.ndarray       # [E, L, 2I, R]


def make_moe(seed: int, *, T: int, H: int, E: int, top_k: int, I: int, R: int, L: int,
             neg_frac: float = 0.05, scale: float = 1.0, name: str = "custom MoE") -> MoeCase:
    """Routed-MoE gemm1 inputs.  Each token gets `top_k` distinct experts drawn
    uniformly without replacement (kept in draw order); lora_ids uniform over
    0..L-1, then -1 with probability `neg_frac`.  A ~ N(0, 1/H), B ~ N(0, 1/R)."""
    rng = np.random.default_rng(seed)
    topk = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :top_k].astype(np.int32)
    lora = rng.integers(0, L, size=T)
    if neg_frac > 0:
        lora = np.where(rng.random(T) < neg_frac, -1, lora)
    lora = lora.astype(np.int32)
    sa, sb = 1.0 / np.sqrt(H), 1.0 / np.sqrt(R)
    a_gate = _normal_bf16(rng, (E, L, R, H), sa)
    a_up = _normal_bf16(rng, (E, L, R, H), sa)
    b_gate = _normal_bf16(rng, (E, L, I, R), sb)
    b_up = _normal_bf16(rng, (E, L, I, R), sb)
    a_shared = _normal_bf16(rng, (E, L, R, H), sa)
    b_fused = _normal_bf16(rng, (E, L, 2 * I, R), sb)
    x = _normal_bf16(rng, (T, H), 1.0)
    return MoeCase(name, T, H, E, top_k, I, R, L, float(scale), np.ascontiguousarray(topk),
                   np.ascontiguousarray(lora), x, a_gate, a_up, b_gate, b_up, a_shared, b_fused)


def moe_gemm1(seed: int = 5) -> MoeCase:
    """T=2048 tokens, H=4096, 64 experts, top_k 8, I=1408, rank 16, 8 adapters,
    5% of tokens unadapted, scale 1."""
    return make_moe(seed, T=2048, H=4096, E=64, top_k=8, I=1408, R=16, L=8,
                    name="MoE gemm1 T=2048 H=4096 E=64 top8 I=1408 R=16 L=8")


# ---------------------------------------------------------------- MoE w2 (down) case
@dataclass
class MoeW2Case:
    name: str
    T: int
    H: int
    E: int
    top_k: int
    I: int
    R: int
    L: int
    scale: float
    topk_ids: np.ndarray      # [T, top_k] int32
    lora_ids: np.ndarray      # [T] int32, -1 = none
    topk_weights: np.ndarray  # [T, top_k] float32, each token's weights sum to 1
    x2: np.ndarray            # [T*top_k, I] uint16: the activation fed to the down projection
    a_down: np.ndarray        # [E, L, R, I]
    b_down: np.ndarray        # [E, L, H, R]
    y: np.ndarray             # [T*top_k, H] uint16: the per-pair down-projection output


def make_moe_w2(seed: int, *, T: int, H: int, E: int, top_k: int, I: int, R: int, L: int,
                neg_frac: float = 0.05, scale: float = 1.0, name: str = "custom MoE w2") -> MoeW2Case:
    """Routed-MoE down-projection inputs, routed like make_moe.  Routing
    weights are uniform draws normalized per token; x2 and y ~ N(0, 1);
    A ~ N(0, 1/I), B ~ N(0, 1/R)."""
    rng = np.random.default_rng(seed)
    topk = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :top_k].astype(np.int32)
    lora = rng.integers(0, L, size=T)
    if neg_frac > 0:
        lora = np.where(rng.random(T) < neg_frac, -1, lora)
    lora = lora.astype(np.int32)
    w = rng.random((T, top_k), dtype=np.float32) + np.float32(0.05)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    a_down = _normal_bf16(rng, (E, L, R, I), 1.0 / np.sqrt(I))
    b_down = _normal_bf16(rng, (E, L, H, R), 1.0 / np.sqrt(R))
    x2 = _normal_bf16(rng, (T * top_k, I), 1.0)
    y = _normal_bf16(rng, (T * top_k, H), 1.0)
    return MoeW2Case(name, T, H, E, top_k, I, R, L, float(scale), np.ascontiguousarray(topk),
                     np.ascontiguousarray(lora), np.ascontiguousarray(w), x2, a_down, b_down, y)


def moe_w2(seed: int = 6) -> MoeW2Case:
    """The down projection of the MoE gemm1 model: T=2048, H=4096, 64 experts,
    top_k 8, I=1408, rank 16, 8 adapters, 5% of tokens unadapted, scale 1."""
    return make_moe_w2(seed, T=2048, H=4096, E=64, top_k=8, I=1408, R=16, L=8,
                       name="MoE w2 T=2048 H=4096 E=64 top8 I=1408 R=16 L=8")


@dataclass
class ExpertFoldCase:
    name: str
    E: int
    n: int                     # sorted (expanded) rows
    k_in: int
    n_out: int
    R: int
    num_slots: int             # pairs in the pool (one per adapted expert)
    expert_offsets: np.ndarray  # [E + 1] uint32 prefix sum of rows per expert
    adapted: np.ndarray        # [num_slots] uint16 adapted experts, in pool-slot order
    expert_slot: np.ndarray    # [E] int32 pool slot of each expert's pair, -1 = none
    x: np.ndarray              # [n, k_in] uint16 sorted input
    y: np.ndarray              # [n, n_out] uint16 sorted output (folded in place)
    a_pool: np.ndarray         # [num_slots, 1, R, k_in]
    b_pool: np.ndarray         # [num_slots, n_out, R]
    scale: np.ndarray          # [num_slots] float32


def make_expert_fold(seed: int, *, T: int, top_k: int, E: int, k_in: int, n_out: int, R: int,
                     adapted_frac: float = 0.75, scale: float = 2.0,
                     name: str = "custom expert fold") -> ExpertFoldCase:
    """Expert-sorted rows of a routed MoE batch: each of T tokens picks top_k
    distinct experts uniformly, expert e's rows are its tokens' copies
    (expert_offsets is the prefix sum of the per-expert counts), and a random
    `adapted_frac` of the experts has a pair (A ~ N(0, 1/k_in), B ~ N(0, 1/R))
    at a random pool slot.  x, y ~ N(0, 1).  With T = n and E = 1, top_k = 1
    it is the router fold's one block of all rows."""
    rng = np.random.default_rng(seed)
    topk = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :top_k]
    counts = np.bincount(topk.reshape(-1), minlength=E)
    off = np.zeros(E + 1, np.uint32)
    off[1:] = np.cumsum(counts)
    n = int(off[-1])
    n_ad = max(1, int(round(adapted_frac * E)))
    adapted = rng.permutation(E)[:n_ad].astype(np.uint16)
    slot = np.full(E, -1, np.int32)
    slot[adapted.astype(np.int64)] = np.arange(n_ad, dtype=np.int32)
    a_pool = _normal_bf16(rng, (n_ad, 1, R, k_in), 1.0 / np.sqrt(k_in))
    b_pool = _normal_bf16(rng, (n_ad, n_out, R), 1.0 / np.sqrt(R))
    x = _normal_bf16(rng, (n, k_in), 1.0)
    y = _normal_bf16(rng, (n, n_out), 1.0)
    return ExpertFoldCase(name, E, n, k_in, n_out, R, n_ad, off, adapted, slot, x, y, a_pool, b_pool,
                          np.full(n_ad, scale, np.float32))


def expert_fold(seed: int = 7) -> ExpertFoldCase:
    """The gate_up projection of the MoE model in its expert-sorted layout:
    T=2048 tokens, top_k 8 (16384 sorted rows), 64 experts of which 48 have a
    pair, k_in 4096, n_out 2816 (2 x 1408), rank 16."""
    return make_expert_fold(seed, T=2048, top_k=8, E=64, k_in=4096, n_out=2816, R=16,
                            name="expert-sorted fold T=2048 top8 E=64 k_in=4096 n_out=2816 R=16")


def router_fold(seed: int = 8) -> ExpertFoldCase:
    """Router LoRA: 2048 tokens, hidden 4096, gate logits over 64 experts, rank 16."""
    return make_expert_fold(seed, T=2048, top_k=1, E=1, k_in=4096, n_out=64, R=16, adapted_frac=1.0,
                            name="router fold n=2048 hidden=4096 E=64 R=16")


CONFIGS = {1: tiny_bgmv, 2: decode_bgmv, 3: prefill_sgmv, 4: no_reuse, 5: moe_gemm1}


# ---------------------------------------------------------------- save / load
_CASE_TYPES = {cls.__name__: cls for cls in (DenseCase, MoeCase, MoeW2Case, ExpertFoldCase)}


def save_case(case, path: str) -> None:
    """Write a case to an .npz file: its arrays as arrays, every other field
    (sizes, name, slice sizes, the meta dict) as one JSON string.  Nothing in
    the file needs pickle to read back."""
    import dataclasses
    import json
    arrays, plain = {}, {}
    for f in dataclasses.fields(case):
        v = getattr(case, f.name)
        if isinstance(v, np.ndarray):
            arrays[f.name] = v
        elif isinstance(v, dict):      # DenseCase.meta: arrays (sequence lengths, slots)
            plain[f.name] = {}
            for k, e in v.items():
                arrays[f"{f.name}.{k}"] = np.asarray(e)
        else:
            plain[f.name] = list(v) if isinstance(v, tuple) else v
    np.savez(path, __case__=np.array(json.dumps({"type": type(case).__name__, "fields": plain})), **arrays)


def load_case(path: str):
    """Read a case written by save_case (numpy's loader with pickle disabled)."""
    import json
    with np.load(path, allow_pickle=False) as z:
        head = json.loads(str(z["__case__"]))
        cls = _CASE_TYPES[head["type"]]
        kw = dict(head["fields"])
        for k in z.files:
            if k == "__case__":
                continue
            if "." in k:
                d, e = k.split(".", 1)
                kw.setdefault(d, {})[e] = np.ascontiguousarray(z[k])
            else:
                kw[k] = np.ascontiguousarray(z[k])
    if "slice_sizes" in kw:
        kw["slice_sizes"] = tuple(kw["slice_sizes"])
    return cls(**kw)
