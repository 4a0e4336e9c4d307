"""CPU checks of the benchmark's byte accounting: the algorithmic bytes that
the roofline figures divide by, recomputed here term by term from the
workload definitions (no GPU needed)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tenant_lora_serving_amd import inputs as I  # noqa: E402


def test_decode_bytes_term_by_term():
    c = I.decode_bgmv()
    act = (c.slot >= 0) & (c.slot < c.num_slots)
    rows = int(act.sum())
    slots = set(int(s) for s in c.slot[act])
    x = rows * c.k_in * 2
    a = len(slots) * c.num_slices * c.max_rank * c.k_in * 2
    b = len(slots) * c.n_out * c.max_rank * 2
    y = rows * c.n_out * 2 * 2
    assert bench.algorithmic_bytes(c) == x + a + b + y
    # the decode batch the bench line quotes: 242 adapted rows over 31 adapters
    assert (rows, len(slots)) == (242, 31)
    assert x + a + b + y == 26214400


def test_moe_bytes_by_brute_force_over_pairs():
    c = I.moe_gemm1()
    E, L, R, H, I_ = c.E, c.L, c.R, c.H, c.I
    touched, t_act, pairs = set(), 0, 0
    for t in range(c.T):
        l = int(c.lora_ids[t])
        if 0 <= l < L:
            t_act += 1
        for j in range(c.top_k):
            e = int(c.topk_ids[t, j])
            pairs += 1
            if 0 <= l < L and 0 <= e < E:
                touched.add((l, e))
    regular = t_act * H * 2 + len(touched) * (2 * R * H + 2 * I_ * R) * 2 + pairs * 2 * I_ * 2
    shared = t_act * H * 2 + len(touched) * (R * H + 2 * I_ * R) * 2 + pairs * 2 * I_ * 2
    assert bench.moe_bytes(c.topk_ids, c.lora_ids, L, E, 2 * R * H, 2 * I_ * R, H * 2, 2 * I_ * 2, True) == regular
    assert bench.moe_bytes(c.topk_ids, c.lora_ids, L, E, R * H, 2 * I_ * R, H * 2, 2 * I_ * 2, True) == shared


def test_w2_bytes_by_brute_force_over_pairs():
    c = I.make_moe_w2(3, T=40, H=64, E=5, top_k=3, I=24, R=8, L=2)
    c.lora_ids[3] = 7                      # an invalid adapter id
    c.topk_ids[5, 1] = 9                   # an invalid expert id
    touched, valid = set(), 0
    for t in range(c.T):
        for j in range(c.top_k):
            l, e = int(c.lora_ids[t]), int(c.topk_ids[t, j])
            if 0 <= l < c.L and 0 <= e < c.E:
                valid += 1
                touched.add((l, e))
    exp = valid * (c.I * 2 + c.H * 4) + len(touched) * (c.R * c.I + c.H * c.R) * 2
    got = bench.moe_bytes(c.topk_ids, c.lora_ids, c.L, c.E, c.R * c.I, c.H * c.R, c.I * 2, c.H * 4, False)
    assert got == exp


def test_one_gpu_only():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode != 0 and "one GPU" in r.stderr
