"""Pins of the fp64 CPU oracle against facts fixed outside it.

Each check here is one of: a small example worked by hand (expected numbers
derived in the comments), a special case that reduces to a library routine
(numpy matmul, Python's sorted), brute force over tiny inputs, or an
invariant the definitions imply.  None of them re-types the oracle's own
loops.  tests/test_oracle_mutants.py plants plausible mistakes in a copy of
the oracle and checks that these pins catch each one.

Definitions pinned (pages cited by title and section):
  vLLM punica_base.py, PunicaWrapperBase.add_shrink / add_expand semantics;
  metrale lora_delta docs: apply_lora_bgmv, LoraPair, module invariants;
  FlashInfer bgmv_moe_gemm1_lora_delta: formula, shared-A form, parameters.
"""
import itertools

import numpy as np
import pytest

from oracle import oracle as O
from tenant_lora_serving_amd import inputs as I

bits = I.f32_to_bf16_bits
f32 = I.bf16_bits_to_f32


def b16(a):
    """bf16 bit patterns of values that are exactly representable."""
    a = np.asarray(a, dtype=np.float32)
    out = bits(a)
    assert np.array_equal(f32(out), a), "hand values must be exact in bf16"
    return out


# ============================================================== metadata pins
def test_meta_hand_example():
    # slot = [2, -1, 0, 2, 5, 0, 1], S = 4.  Row 1 has no adapter, row 4 names
    # slot 5 >= S (invalid).  Active rows by (slot, row): slot 0 -> rows 2, 5;
    # slot 1 -> row 6; slot 2 -> rows 0, 3.
    rows, offs, sl, cnt = O.meta_build(np.array([2, -1, 0, 2, 5, 0, 1]), 4)
    assert rows.tolist() == [2, 5, 6, 0, 3]
    assert offs.tolist() == [0, 2, 3, 5]
    assert sl.tolist() == [0, 1, 2]
    assert cnt.tolist() == [5, 3, 1, 0]


def test_meta_hand_long_segment():
    # 20 rows alternating slot 1 / slot 0 except rows 0..3 which are -1:
    # rows 4..19 -> 16 rows; even rows slot 1 (8 rows), odd rows slot 0 (8).
    # Then append 17 rows of slot 3 -> one segment of 17 >= 16 rows.
    slot = [-1] * 4 + [1 if i % 2 == 0 else 0 for i in range(4, 20)] + [3] * 17
    rows, offs, sl, cnt = O.meta_build(np.array(slot), 4)
    assert rows.tolist() == list(range(5, 20, 2)) + list(range(4, 20, 2)) + list(range(20, 37))
    assert offs.tolist() == [0, 8, 16, 33]
    assert sl.tolist() == [0, 1, 3]
    assert cnt.tolist() == [33, 3, 0, 1]


def _meta_by_python_sort(slot, S):
    act = [i for i, s in enumerate(slot) if 0 <= s < S]
    act = sorted(act, key=lambda i: (slot[i], i))
    offs, sl, nlong = [], [], 0
    pos = 0
    for s, grp in itertools.groupby(act, key=lambda i: slot[i]):
        g = list(grp)
        offs.append(pos)
        sl.append(s)
        nlong += len(g) >= 16
        pos += len(g)
    offs.append(pos)
    ninv = sum(1 for s in slot if s >= S)
    return act, offs, sl, [len(act), len(sl), ninv, nlong]


def test_meta_brute_force_python_sort():
    rng = np.random.default_rng(11)
    for trial in range(400):
        n = int(rng.integers(0, 90))
        S = int(rng.integers(1, 12))
        slot = rng.integers(-3, S + 3, size=n).astype(np.int32)
        if trial % 7 == 0:
            slot[:] = rng.integers(0, S)            # one long segment
        got = O.meta_build(slot, S)
        exp = _meta_by_python_sort(slot.tolist(), S)
        assert got[0].tolist() == exp[0]
        assert got[1].tolist() == exp[1]
        assert got[2].tolist() == exp[2]
        assert got[3].tolist() == exp[3]


def test_meta_structure_large():
    rng = np.random.default_rng(12)
    slot = rng.integers(-2, 40, size=5000).astype(np.int32)
    rows, offs, sl, cnt = O.meta_build(slot, 37)
    act = np.flatnonzero((slot >= 0) & (slot < 37))
    assert sorted(rows.tolist()) == act.tolist()                 # a permutation of active rows
    assert np.all(np.diff(offs) > 0) and offs[0] == 0 and offs[-1] == cnt[0]
    assert np.all(np.diff(sl) > 0)
    for g in range(len(sl)):
        seg = rows[offs[g]:offs[g + 1]]
        assert np.all(slot[seg] == sl[g]) and np.all(np.diff(seg) > 0)
    assert cnt[2] == int((slot >= 37).sum())


def test_moe_keys_hand():
    # E = 4 experts, L = 2 adapters, top_k = 2.
    # token 0: lora 1, experts (3, 0) -> keys 1*4+3 = 7, 1*4+0 = 4
    # token 1: lora -1            -> -1, -1
    # token 2: lora 2 (>= L)      -> invalid = L*E = 8 for both
    # token 3: lora 0, experts (4, -2) both out of [0, 4) -> 8, 8
    # token 4: lora 0, experts (2, 1) -> 2, 1
    topk = np.array([[3, 0], [1, 2], [0, 1], [4, -2], [2, 1]])
    lora = np.array([1, -1, 2, 0, 0])
    assert O.moe_keys(topk, lora, 4, 2).tolist() == [7, 4, -1, -1, 8, 8, 8, 8, 2, 1]


# ============================================================== dense delta pins
def _hand_case():
    """Two slots, two slices (widths 2 and 1), k_in = 2, max_rank = 2.

    Row 0 uses slot 1; row 1 has no adapter (slot -1).
      x0 = [1, 2]
      slot 1, slice 0: A = [[1, 0], [0.5, 1]]  -> x0.A^T = [1, 2.5];  scale 2 -> xa0 = [2, 5]
      slot 1, slice 1: A = [[0, 1], [1, 1]]    -> x0.A^T = [2, 3];    scale 2 -> xa1 = [4, 6]
      slot 1, B rows (N = 3): [[1, 0], [0, 1], [1, -1]]
        slice 0 cols 0,1: [2*1 + 5*0, 2*0 + 5*1] = [2, 5]
        slice 1 col 2:    4*1 + 6*(-1)           = -2
      y0 = [0.5, 0.25, -1]  -> y0' = [2.5, 5.25, -3]
    Slot 0 is filled with large values so that reading the wrong slot shows.
    """
    x = b16([[1, 2], [3, -1]])
    a = np.zeros((2, 2, 2, 2), np.float32)
    a[0] = 3.0
    a[1, 0] = [[1, 0], [0.5, 1]]
    a[1, 1] = [[0, 1], [1, 1]]
    b = np.zeros((2, 3, 2), np.float32)
    b[0] = 7.0
    b[1] = [[1, 0], [0, 1], [1, -1]]
    scale = np.array([10.0, 2.0], np.float32)
    y = b16([[0.5, 0.25, -1], [7, 8, 9]])
    slot = np.array([1, -1], np.int32)
    return x, b16(a), b16(b), scale, y, slot


def test_dense_hand_example():
    x, a, b, scale, y, slot = _hand_case()
    xa = O.shrink_rows(x, 2, a, scale, 2, 2, 2, slot, [0, 1])
    assert xa[0].tolist() == [[2.0, 5.0], [4.0, 6.0]]
    assert np.isnan(xa[1]).all()                       # inactive row left unwritten
    out = O.fused_rows(x, 2, a, b, scale, 2, (2, 1), 2, slot, [0, 1], y)
    assert out.tolist() == [[2.5, 5.25, -3.0], [7.0, 8.0, 9.0]]


def test_dense_hand_add_inputs_and_offset():
    x, a, b, scale, y, slot = _hand_case()
    xa = O.shrink_rows(x, 2, a, scale, 2, 2, 2, slot, [0, 1])
    xa = np.nan_to_num(xa)
    # add_inputs = 0: the window is overwritten with the delta
    out = O.expand_rows(xa, b, 2, (2, 1), 2, slot, [0, 1], y, 0, add_inputs=False)
    assert out.tolist() == [[2.0, 5.0, -2.0], [7.0, 8.0, 9.0]]
    # offset_start = 1 on a 5-wide y: columns 1..3 get the delta, 0 and 4 keep theirs
    y5 = b16([[1, 1, 1, 1, 1], [2, 2, 2, 2, 2]])
    out = O.expand_rows(xa, b, 2, (2, 1), 2, slot, [0, 1], y5, 1, add_inputs=True)
    assert out.tolist() == [[1.0, 3.0, 6.0, -1.0, 1.0], [2.0] * 5]


def _random_case(seed, n=40, k_in=64, slices=(24, 8, 16), S=5, R=8, neg=True):
    rng = np.random.default_rng(seed)
    slot = rng.integers(-1 if neg else 0, S, size=n).astype(np.int32)
    return I.make_dense(seed, n=n, k_in=k_in, slice_sizes=slices, num_slots=S, max_rank=R,
                        rank_choices=[R // 2, R], slot=slot, scale_num=16.0)


def _per_slot_matmul(c, y_in=None, offset_start=0, add_inputs=True):
    """SGMV as one library GEMM pair per slot: for the rows of slot s,
    Y[:, window] (+)= scale_s * (X @ A_s^T) @ B_s^T (numpy float64 matmul)."""
    X = f32(c.x).astype(np.float64)
    Y = f32(c.y if y_in is None else y_in).astype(np.float64)
    out = Y.copy()
    off = np.concatenate([[0], np.cumsum(c.slice_sizes)])
    for s in range(c.num_slots):
        rows = np.flatnonzero(c.slot == s)
        if rows.size == 0:
            continue
        for l in range(c.num_slices):
            A = f32(c.a_pool[s, l]).astype(np.float64)            # [R, k]
            Bl = f32(c.b_pool[s, off[l]:off[l + 1]]).astype(np.float64)   # [w, R]
            d = np.matmul(np.matmul(X[rows], A.T) * float(c.scale[s]), Bl.T)
            cols = slice(offset_start + off[l], offset_start + off[l + 1])
            out[rows, cols] = (Y[rows, cols] if add_inputs else 0.0) + d
    return out


def test_dense_per_slot_library_gemm():
    for seed in range(6):
        c = _random_case(100 + seed)
        got = O.case_fused_rows(c, np.arange(c.n))
        exp = _per_slot_matmul(c)
        np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_dense_single_slot_closed_form():
    # every row on one slot: y + s * (x A^T) B^T with a single slice
    c = I.make_dense(7, n=33, k_in=128, slice_sizes=(40,), num_slots=3, max_rank=16,
                     rank_choices=[16], slot=np.full(33, 2, np.int32), scale_num=8.0)
    got = O.case_fused_rows(c, np.arange(c.n))
    X, Y = f32(c.x).astype(np.float64), f32(c.y).astype(np.float64)
    A, B = f32(c.a_pool[2, 0]).astype(np.float64), f32(c.b_pool[2]).astype(np.float64)
    exp = Y + float(c.scale[2]) * (X @ A.T) @ B.T
    np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_dense_materialized_weight_brute_force():
    # Different association: W_s = scale_s * B_s A_s as a dense [N, k] matrix,
    # then y_i + W_s x_i for each row (the whole-matrix brute force).
    c = I.tiny_bgmv()
    got = O.case_fused_rows(c, np.arange(c.n))
    X, Y = f32(c.x).astype(np.float64), f32(c.y).astype(np.float64)
    for i in range(c.n):
        s = int(c.slot[i])
        if s < 0:
            assert np.array_equal(got[i], Y[i])
            continue
        W = float(c.scale[s]) * f32(c.b_pool[s]).astype(np.float64) @ f32(c.a_pool[s, 0]).astype(np.float64)
        exp = Y[i] + W @ X[i]
        np.testing.assert_allclose(got[i], exp, rtol=1e-12, atol=1e-12)


def test_dense_negative_and_invalid_slot_exact():
    c = _random_case(21, n=30, S=4)
    c.slot[::3] = -1
    c.slot[1::7] = 9            # >= S: excluded
    got = O.case_fused_rows(c, np.arange(c.n))
    Y = f32(c.y).astype(np.float64)
    off = (c.slot < 0) | (c.slot >= c.num_slots)
    assert off.any()
    assert np.array_equal(got[off], Y[off])


def test_dense_zero_scale_and_zero_pool_exact():
    c = _random_case(22)
    Y = f32(c.y).astype(np.float64)
    assert np.array_equal(O.fused_rows(c.x, c.k_in, c.a_pool, c.b_pool, c.scale * 0,
                                       c.num_slots, c.slice_sizes, c.max_rank, c.slot,
                                       np.arange(c.n), c.y), Y)
    c.a_pool[:] = 0
    assert np.array_equal(O.case_fused_rows(c, np.arange(c.n)), Y)


def test_dense_rank_padding_changes_nothing():
    # Re-pack the same adapters at max_rank 16 instead of 8 (zero pad rows of
    # A and pad columns of B): the result is bitwise identical.
    c = _random_case(23, R=8)
    got8 = O.case_fused_rows(c, np.arange(c.n))
    a16 = np.zeros(c.a_pool.shape[:2] + (16, c.k_in), np.uint16)
    a16[:, :, :8] = c.a_pool
    b16_ = np.zeros(c.b_pool.shape[:2] + (16,), np.uint16)
    b16_[:, :, :8] = c.b_pool
    got16 = O.fused_rows(c.x, c.k_in, a16, b16_, c.scale, c.num_slots, c.slice_sizes, 16,
                         c.slot, np.arange(c.n), c.y)
    assert np.array_equal(got8, got16)


def test_dense_row_permutation_and_slot_relabel():
    c = _random_case(24)
    base = O.case_fused_rows(c, np.arange(c.n))
    perm = np.random.default_rng(0).permutation(c.n)
    got = O.fused_rows(c.x[perm], c.k_in, c.a_pool, c.b_pool, c.scale, c.num_slots,
                       c.slice_sizes, c.max_rank, c.slot[perm], np.arange(c.n), c.y[perm])
    assert np.array_equal(got, base[perm])
    relabel = np.random.default_rng(1).permutation(c.num_slots)   # new slot of old slot s
    inv = np.argsort(relabel)
    slot2 = np.where(c.slot >= 0, relabel[np.maximum(c.slot, 0)], c.slot).astype(np.int32)
    got = O.fused_rows(c.x, c.k_in, c.a_pool[inv], c.b_pool[inv], c.scale[inv], c.num_slots,
                       c.slice_sizes, c.max_rank, slot2, np.arange(c.n), c.y)
    assert np.array_equal(got, base)


def test_dense_scale_doubling_doubles_delta():
    c = _random_case(25)
    rows = np.arange(c.n)
    xa1 = np.nan_to_num(O.shrink_rows(c.x, c.k_in, c.a_pool, c.scale, c.num_slots,
                                      c.num_slices, c.max_rank, c.slot, rows))
    xa2 = np.nan_to_num(O.shrink_rows(c.x, c.k_in, c.a_pool, c.scale * 2, c.num_slots,
                                      c.num_slices, c.max_rank, c.slot, rows))
    d1 = O.expand_rows(xa1, c.b_pool, c.num_slots, c.slice_sizes, c.max_rank, c.slot, rows,
                       np.zeros_like(c.y), 0, add_inputs=False)
    d2 = O.expand_rows(xa2, c.b_pool, c.num_slots, c.slice_sizes, c.max_rank, c.slot, rows,
                       np.zeros_like(c.y), 0, add_inputs=False)
    assert np.array_equal(d2, 2 * d1)
    assert np.abs(d1).max() > 0


def test_dense_row_subset_matches_full():
    c = _random_case(26)
    full = O.case_fused_rows(c, np.arange(c.n))
    sub = [5, 0, 17, 5, 39]
    assert np.array_equal(O.case_fused_rows(c, sub), full[sub])


# ============================================================== MoE pins
def _small_moe(seed=31, T=12, H=64, E=5, top_k=3, I_=24, R=8, L=3, neg_frac=0.25):
    return I.make_moe(seed, T=T, H=H, E=E, top_k=top_k, I=I_, R=R, L=L, neg_frac=neg_frac,
                      scale=0.5)


def _moe_library(case, shared):
    """Per pair, the page's formula with numpy matmul on the bank matrices."""
    X = f32(case.x).astype(np.float64)
    out = np.zeros((case.T * case.top_k, 2 * case.I))
    for t in range(case.T):
        l = int(case.lora_ids[t])
        for j in range(case.top_k):
            e = int(case.topk_ids[t, j])
            if l < 0 or l >= case.L or e < 0 or e >= case.E:
                continue
            if shared:
                A = f32(case.a_shared[e, l]).astype(np.float64)
                B = f32(case.b_fused[e, l]).astype(np.float64)
                d = case.scale * (B @ (A @ X[t]))
            else:
                g = f32(case.b_gate[e, l]).astype(np.float64) @ (f32(case.a_gate[e, l]).astype(np.float64) @ X[t])
                u = f32(case.b_up[e, l]).astype(np.float64) @ (f32(case.a_up[e, l]).astype(np.float64) @ X[t])
                d = case.scale * np.concatenate([g, u])
            out[t * case.top_k + j] = d
    return out


@pytest.mark.parametrize("shared", [False, True])
def test_moe_library_formula(shared):
    c = _small_moe()
    got = O.case_moe_pairs(c, shared, np.arange(c.T * c.top_k))
    np.testing.assert_allclose(got, _moe_library(c, shared), rtol=1e-12, atol=1e-12)


def test_moe_skipped_and_invalid_pairs_are_zero():
    c = _small_moe()
    c.lora_ids[0] = -1
    c.lora_ids[1] = c.L            # invalid adapter
    c.lora_ids[2] = c.lora_ids[3] = 1
    c.topk_ids[2, 0] = 0
    c.topk_ids[2, 1] = c.E         # invalid expert
    c.topk_ids[3, 0] = -4
    got = O.case_moe_pairs(c, False, np.arange(c.T * c.top_k))
    k = c.top_k
    for p in list(range(0, k)) + list(range(k, 2 * k)) + [2 * k + 1, 3 * k]:
        assert not got[p].any()
    assert got[2 * k].any()


def test_moe_shared_equals_regular_when_a_is_shared():
    c = _small_moe(neg_frac=0.1)
    c.a_gate[:] = c.a_shared
    c.a_up[:] = c.a_shared
    c.b_gate[:] = c.b_fused[:, :, :c.I]
    c.b_up[:] = c.b_fused[:, :, c.I:]
    pairs = np.arange(c.T * c.top_k)
    assert np.array_equal(O.case_moe_pairs(c, False, pairs), O.case_moe_pairs(c, True, pairs))


def test_moe_equals_dense_on_expanded_rows():
    # x_exp[t*top_k + j] = x[t], slot = l*E + e over a pool of L*E adapters with
    # two slices (I, I), zero base y and scale 1: the MoE delta is the dense delta.
    c = _small_moe(neg_frac=0.2)
    c.scale = 1.0
    T, k, E, L, R, H, I_ = c.T, c.top_k, c.E, c.L, c.R, c.H, c.I
    x_exp = np.repeat(c.x, k, axis=0)
    key = np.where(np.repeat(c.lora_ids, k) >= 0,
                   np.repeat(c.lora_ids, k) * E + c.topk_ids.reshape(-1), -1).astype(np.int32)
    a_pool = np.zeros((L * E, 2, R, H), np.uint16)
    b_pool = np.zeros((L * E, 2 * I_, R), np.uint16)
    for l in range(L):
        for e in range(E):
            a_pool[l * E + e, 0], a_pool[l * E + e, 1] = c.a_gate[e, l], c.a_up[e, l]
            b_pool[l * E + e, :I_], b_pool[l * E + e, I_:] = c.b_gate[e, l], c.b_up[e, l]
    dense = O.fused_rows(x_exp, H, a_pool, b_pool, np.ones(L * E, np.float32), L * E, (I_, I_),
                         R, key, np.arange(T * k), np.zeros((T * k, 2 * I_), np.uint16))
    moe = O.case_moe_pairs(c, False, np.arange(T * k))
    assert np.array_equal(dense, moe)


def test_moe_single_expert_top1_is_bgmv():
    # E = 1, top_k = 1: token t's pair is a dense row with slot lora_ids[t]
    c = _small_moe(E=1, top_k=1, L=4, neg_frac=0.2)
    c.scale = 1.0
    a_pool = np.stack([np.stack([c.a_gate[0, l], c.a_up[0, l]]) for l in range(c.L)])
    b_pool = np.stack([np.concatenate([c.b_gate[0, l], c.b_up[0, l]]) for l in range(c.L)])
    dense = O.fused_rows(c.x, c.H, a_pool, b_pool, np.ones(c.L, np.float32), c.L, (c.I, c.I),
                         c.R, c.lora_ids, np.arange(c.T), np.zeros((c.T, 2 * c.I), np.uint16))
    assert np.array_equal(dense, O.case_moe_pairs(c, False, np.arange(c.T)))


# ============================================================== MoE w2 (down) pins
def _small_w2(seed=41, T=10, H=48, E=4, top_k=3, I_=40, R=8, L=3, neg_frac=0.25):
    return I.make_moe_w2(seed, T=T, H=H, E=E, top_k=top_k, I=I_, R=R, L=L, neg_frac=neg_frac,
                         scale=0.5)


def _w2_library(case, weighted):
    """Per pair, the delta written with numpy matmul on the bank matrices."""
    X2 = f32(case.x2).astype(np.float64)
    out = f32(case.y).astype(np.float64).copy()
    for t in range(case.T):
        l = int(case.lora_ids[t])
        for j in range(case.top_k):
            e = int(case.topk_ids[t, j])
            if l < 0 or l >= case.L or e < 0 or e >= case.E:
                continue
            p = t * case.top_k + j
            A = f32(case.a_down[e, l]).astype(np.float64)
            B = f32(case.b_down[e, l]).astype(np.float64)
            w = float(case.topk_weights[t, j]) if weighted else 1.0
            out[p] += w * case.scale * (B @ (A @ X2[p]))
    return out


@pytest.mark.parametrize("weighted", [False, True])
def test_w2_library_formula(weighted):
    c = _small_w2()
    got = O.case_moe_w2_pairs(c, np.arange(c.T * c.top_k), weighted)
    np.testing.assert_allclose(got, _w2_library(c, weighted), rtol=1e-12, atol=1e-12)


def test_w2_unrouted_pairs_keep_y_exactly():
    c = _small_w2()
    c.lora_ids[0] = -1
    c.lora_ids[1] = c.L            # invalid adapter
    c.lora_ids[2] = c.lora_ids[3] = 1
    c.topk_ids[2, 0] = 0
    c.topk_ids[2, 1] = c.E         # invalid expert
    c.topk_ids[3, 0] = -4
    got = O.case_moe_w2_pairs(c, np.arange(c.T * c.top_k))
    y = f32(c.y).astype(np.float64)
    k = c.top_k
    for p in list(range(0, 2 * k)) + [2 * k + 1, 3 * k]:
        assert np.array_equal(got[p], y[p])
    assert not np.array_equal(got[2 * k], y[2 * k])


def test_w2_unit_weights_equal_unweighted_and_weights_scale_the_delta():
    c = _small_w2(neg_frac=0.1)
    pairs = np.arange(c.T * c.top_k)
    c.topk_weights[:] = 1.0
    assert np.array_equal(O.case_moe_w2_pairs(c, pairs, True), O.case_moe_w2_pairs(c, pairs, False))
    c.y[:] = 0
    one = O.case_moe_w2_pairs(c, pairs, True)
    c.topk_weights[:] = 2.0
    assert np.array_equal(O.case_moe_w2_pairs(c, pairs, True), 2.0 * one)   # exact in fp64


def test_w2_equals_dense_on_expanded_rows():
    # row p = t*top_k + j is a dense row with slot l*E + e over a pool of L*E
    # adapters with one slice of width H: unweighted, the w2 delta is the dense delta
    c = _small_w2(neg_frac=0.2)
    T, k, E, L, R, H, I_ = c.T, c.top_k, c.E, c.L, c.R, c.H, c.I
    lk = np.repeat(c.lora_ids, k)
    key = np.where(lk >= 0, lk * E + c.topk_ids.reshape(-1), -1).astype(np.int32)
    a_pool = np.zeros((L * E, 1, R, I_), np.uint16)
    b_pool = np.zeros((L * E, H, R), np.uint16)
    for l in range(L):
        for e in range(E):
            a_pool[l * E + e, 0], b_pool[l * E + e] = c.a_down[e, l], c.b_down[e, l]
    dense = O.fused_rows(c.x2, I_, a_pool, b_pool, np.full(L * E, c.scale, np.float32), L * E, (H,),
                         R, key, np.arange(T * k), c.y)
    assert np.array_equal(dense, O.case_moe_w2_pairs(c, np.arange(T * k), False))


def test_w2_single_expert_top1_is_bgmv():
    c = _small_w2(E=1, top_k=1, L=4, neg_frac=0.2)
    a_pool = c.a_down[0][:, None]          # [L, 1, R, I]
    b_pool = c.b_down[0]                   # [L, H, R]
    dense = O.fused_rows(c.x2, c.I, a_pool, b_pool, np.full(c.L, c.scale, np.float32), c.L, (c.H,),
                         c.R, c.lora_ids, np.arange(c.T), c.y)
    assert np.array_equal(dense, O.case_moe_w2_pairs(c, np.arange(c.T), False))


# ============================================================ expert-sorted fold pins
def test_expert_workitems_hand_example():
    # 4 experts own sorted rows 0..3, 3..3 (empty), 3..7 and 7..12.  Adapted, in
    # order: 2 -> (2, 3, 4); 0 -> (0, 0, 3); 9 is past the table; 1's block is
    # empty; 3 -> (3, 7, 5).
    got = O.expert_workitems([0, 3, 3, 7, 12], [2, 0, 9, 1, 3])
    assert got == [(2, 3, 4), (0, 0, 3), (3, 7, 5)]


def test_expert_workitems_degenerate():
    assert O.expert_workitems([], [0, 1]) == []          # no table: no experts
    assert O.expert_workitems([5], [0]) == []             # one offset: no experts
    assert O.expert_workitems([0, 4, 9], []) == []        # nothing adapted
    # a block whose end is not past its start is skipped, the next one is not
    assert O.expert_workitems([0, 5, 2, 9], [1, 2]) == [(2, 2, 7)]
    # an expert listed twice gives two items
    assert O.expert_workitems([0, 2, 6], [1, 1]) == [(1, 2, 4), (1, 2, 4)]


def test_expert_workitems_from_counts():
    rng = np.random.default_rng(11)
    for _ in range(20):
        E = int(rng.integers(1, 40))
        c = rng.integers(0, 5, size=E) * (rng.random(E) < 0.7)
        off = np.concatenate([[0], np.cumsum(c)]).astype(np.uint32)
        adapted = rng.permutation(E + 5)[: int(rng.integers(0, E + 5))]
        want = [(int(e), int(c[:e].sum()), int(c[e])) for e in adapted if e < E and c[e] > 0]
        assert O.expert_workitems(off, adapted) == want


def _fold_case(seed=12, **kw):
    args = dict(T=24, top_k=3, E=7, k_in=72, n_out=40, R=8, adapted_frac=0.6)
    args.update(kw)
    return I.make_expert_fold(seed, **args)


def _fold(c, max_rows=None):
    items = O.expert_workitems(c.expert_offsets, c.adapted)
    return O.fold_sorted(c.x, c.k_in, c.y, items, c.expert_slot, c.a_pool, c.b_pool, c.scale,
                         c.num_slots, (c.n_out,), c.R, max_rows)


def test_fold_leaves_unadapted_rows_and_chunking_does_not_matter():
    c = _fold_case()
    whole = _fold(c)
    row_expert = np.repeat(np.arange(c.E), np.diff(c.expert_offsets.astype(np.int64)))
    unadapted = c.expert_slot[row_expert] < 0
    assert unadapted.any() and (~unadapted).any()
    assert np.array_equal(whole[unadapted], f32(c.y[unadapted]).astype(np.float64))
    assert not np.array_equal(whole[~unadapted], f32(c.y[~unadapted]).astype(np.float64))
    for mr in (1, 5):
        assert np.array_equal(_fold(c, mr), whole)


def test_fold_equals_dense_with_per_row_slots():
    # the fold is the dense delta with each sorted row routed to its expert's slot
    c = _fold_case(seed=13, E=9, adapted_frac=0.5)
    row_expert = np.repeat(np.arange(c.E), np.diff(c.expert_offsets.astype(np.int64)))
    slot = c.expert_slot[row_expert].astype(np.int32)
    dense = O.fused_rows(c.x, c.k_in, c.a_pool, c.b_pool, c.scale, c.num_slots, (c.n_out,), c.R, slot,
                         np.arange(c.n), c.y)
    assert np.array_equal(_fold(c), dense)


def test_router_fold_is_one_pair_over_all_rows():
    c = I.make_expert_fold(14, T=30, top_k=1, E=1, k_in=64, n_out=16, R=8, adapted_frac=1.0)
    x = f32(c.x).astype(np.float64)
    A = f32(c.a_pool[0, 0]).astype(np.float64)
    Bm = f32(c.b_pool[0]).astype(np.float64)
    want = f32(c.y).astype(np.float64) + (float(c.scale[0]) * (x @ A.T)) @ Bm.T
    np.testing.assert_allclose(_fold(c), want, rtol=1e-12, atol=1e-12)


# ============================================================ tensor-parallel shard pins
def _tp_case(seed=21, n=20, k_in=96, slices=(48, 32), S=3, R=16):
    return I.make_dense(seed, n=n, k_in=k_in, slice_sizes=slices, num_slots=S, max_rank=R,
                        slot_kind="uniform_neg")


def test_rank_sharded_shrink_is_the_column_block_of_the_full_shrink():
    # column-parallel S-LoRA: A split along the rank; each shard's xa is the
    # matching rank columns of the full xa, exactly
    c = _tp_case()
    rows = np.arange(c.n)
    full = O.shrink_rows(c.x, c.k_in, c.a_pool, c.scale, c.num_slots, c.num_slices, c.max_rank,
                         c.slot, rows)
    tp, rs = 2, c.max_rank // 2
    for r in range(tp):
        a_sh = np.ascontiguousarray(c.a_pool[:, :, r * rs:(r + 1) * rs, :])
        part = O.shrink_rows(c.x, c.k_in, a_sh, c.scale, c.num_slots, c.num_slices, rs, c.slot, rows)
        np.testing.assert_array_equal(part, full[:, :, r * rs:(r + 1) * rs])


def test_k_sharded_shrink_partials_sum_to_the_full_shrink():
    # row-parallel S-LoRA: x and A split along k; the all-reduce of the shards'
    # xa is the full xa (up to the order of the fp64 sum)
    c = _tp_case(seed=22, slices=(40,))
    rows = np.arange(c.n)
    active = (c.slot >= 0) & (c.slot < c.num_slots)
    full = O.shrink_rows(c.x, c.k_in, c.a_pool, c.scale, c.num_slots, 1, c.max_rank, c.slot, rows)
    tp = 4
    ks = c.k_in // tp
    total = np.zeros_like(full)
    for r in range(tp):
        x_sh = np.ascontiguousarray(c.x[:, r * ks:(r + 1) * ks])
        a_sh = np.ascontiguousarray(c.a_pool[..., r * ks:(r + 1) * ks])
        total += O.shrink_rows(x_sh, ks, a_sh, c.scale, c.num_slots, 1, c.max_rank, c.slot, rows)
    np.testing.assert_allclose(total[active], full[active], rtol=1e-12, atol=1e-14)


def test_offset_expand_of_a_column_shard_is_the_slice_of_the_full_expand():
    # row-parallel S-LoRA: B split along the output; shard r adds its columns
    # at offset_start = r * N / tp and leaves every other column alone
    c = _tp_case(seed=23, slices=(64,))
    rows = np.arange(c.n)
    xa = np.random.default_rng(5).standard_normal((c.n, 1, c.max_rank))
    full = O.expand_rows(xa, c.b_pool, c.num_slots, (64,), c.max_rank, c.slot, rows, c.y)
    y = f32(c.y).astype(np.float64)
    tp, ns = 4, 16
    for r in range(tp):
        b_sh = np.ascontiguousarray(c.b_pool[:, r * ns:(r + 1) * ns, :])
        got = O.expand_rows(xa, b_sh, c.num_slots, (ns,), c.max_rank, c.slot, rows, c.y,
                            offset_start=r * ns)
        cols = np.arange(r * ns, (r + 1) * ns)
        np.testing.assert_array_equal(got[:, cols], full[:, cols])
        rest = np.setdiff1d(np.arange(64), cols)
        np.testing.assert_array_equal(got[:, rest], y[:, rest])
