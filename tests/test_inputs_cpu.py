"""CPU checks of the seeded input generator: the same seed gives the same
case, and save_case / load_case round-trip every field bit for bit."""
import dataclasses

import numpy as np

from tenant_lora_serving_amd import inputs as I


def _same(a, b):
    assert type(a) is type(b)
    for f in dataclasses.fields(a):
        va, vb = getattr(a, f.name), getattr(b, f.name)
        if isinstance(va, np.ndarray):
            assert va.dtype == vb.dtype and va.shape == vb.shape and np.array_equal(va, vb), f.name
        elif isinstance(va, dict):
            assert va.keys() == vb.keys() and all(np.array_equal(va[k], vb[k]) for k in va), f.name
        else:
            assert va == vb, (f.name, va, vb)


def test_seeded_cases_repeat():
    _same(I.tiny_bgmv(), I.tiny_bgmv())
    _same(I.make_moe(3, T=9, H=64, E=4, top_k=2, I=16, R=8, L=2),
          I.make_moe(3, T=9, H=64, E=4, top_k=2, I=16, R=8, L=2))


def test_save_load_round_trip(tmp_path):
    cases = [I.tiny_bgmv(),
             I.make_dense(5, n=40, k_in=64, slice_sizes=(16, 24), num_slots=3, max_rank=8,
                          rank_choices=[4, 8], slot_kind="uniform_neg"),
             I.prefill_sgmv(n_seq=3, len_lo=4, len_hi=9, k_in=64, slice_sizes=(32, 32)),
             I.make_moe(3, T=9, H=64, E=4, top_k=2, I=16, R=8, L=2),
             I.make_moe_w2(4, T=7, H=32, E=3, top_k=2, I=24, R=8, L=2),
             I.make_expert_fold(6, T=20, top_k=2, E=5, k_in=32, n_out=16, R=8)]
    for i, c in enumerate(cases):
        p = str(tmp_path / f"case{i}.npz")
        I.save_case(c, p)
        _same(c, I.load_case(p))
