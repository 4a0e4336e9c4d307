"""The oracle's pins must catch plausible mistakes.

Each mutant below is a copy of oracle/oracle.c with one planted mistake (a
transposed operand, a dropped term, a wrong index or offset, a broken order).
Every mutant is compiled on the CPU, and the pin suite in test_oracle_pins.py
is run against it in a child process; at least one pin must fail.  The
mutations keep every access in bounds, so a mutant fails by value, not by
crashing.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "A transposed": (
        "acc += bf(x[(int64_t)i * ldx + k]) * bf(a[k]);",
        "acc += bf(x[(int64_t)i * ldx + k]) * bf(a_pool[((int64_t)s * num_slices + l) * max_rank"
        " * (int64_t)k_in + (int64_t)k * max_rank + r]);"),
    "scale dropped": ("(double)scale[s] * acc;", "acc;"),
    "scale of slot 0": ("(double)scale[s] * acc;", "(double)scale[0] * acc;"),
    "k loop short": ("for (int32_t k = 0; k < k_in; ++k)", "for (int32_t k = 0; k < k_in - 1; ++k)"),
    "B slice offset dropped": ("((int64_t)s * n_out + off + c) * max_rank", "((int64_t)s * n_out + c) * max_rank"),
    "y slice offset dropped": ("const int64_t col = offset_start + off + c;", "const int64_t col = offset_start + c;"),
    "offset_start ignored": ("const int64_t col = offset_start + off + c;", "const int64_t col = off + c;"),
    "add_inputs ignored": ("yo[col] = (add_inputs ? bf(yi[col]) : 0.0) + d;", "yo[col] = bf(yi[col]) + d;"),
    "B transposed": (
        "d += u[r] * bf(b[r]);",
        "d += u[r] * bf(b_pool[(int64_t)s * n_out * max_rank + (int64_t)r * n_out + off + c]);"),
    "rank loop short": ("for (int32_t r = 0; r < max_rank; ++r)\n                    d +=",
                        "for (int32_t r = 0; r < max_rank - 1; ++r)\n                    d +="),
    "meta rows descending": ("for (int32_t i = 0; i < n; ++i)\n            if (slot[i] == s)",
                             "for (int32_t i = n - 1; i >= 0; --i)\n            if (slot[i] == s)"),
    "meta long threshold": ("if (pos - start >= 16)", "if (pos - start > 16)"),
    "meta invalid count": ("if (slot[i] >= num_slots)\n            ++ninvalid;",
                           "if (slot[i] > num_slots)\n            ++ninvalid;"),
    "moe key transposed": ("k = l * num_experts + e;", "k = e * num_loras + l;"),
    "moe gate/up swapped": ("o[(int64_t)sigma * inter + c] = scale * d;",
                            "o[(int64_t)(1 - sigma) * inter + c] = scale * d;"),
    "moe adapter stride dropped": (
        "const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[sigma * num_experts + e]\n"
        "                                    + (int64_t)l * lora_stride_a;",
        "const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[sigma * num_experts + e];"),
    "moe shared B stride dropped": (
        "const uint16_t *B = (const uint16_t *)(intptr_t)w_ptr_b[e] + (int64_t)l * lora_stride_b;",
        "const uint16_t *B = (const uint16_t *)(intptr_t)w_ptr_b[e];"),
    "moe unadapted counted invalid": ("if (l < 0)\n                k = -1;", "if (l < 0)\n                k = S;"),
    "moe unadapted pair not zeroed": ("for (int64_t c = 0; c < width; ++c)\n            o[c] = 0.0;",
                                      "for (int64_t c = 0; c < width; ++c)\n            o[c] = 1.0;"),
    "w2 routing weight ignored": ("const double w = topk_weights ? (double)topk_weights[p] : 1.0;",
                                  "const double w = 1.0;"),
    "w2 weight of token row": ("(double)topk_weights[p] : 1.0;", "(double)topk_weights[t] : 1.0;"),
    "w2 expert of token row": ("const int32_t e = topk_ids[p];\n        const uint16_t *yp",
                               "const int32_t e = topk_ids[t];\n        const uint16_t *yp"),
    "w2 adapter stride dropped": (
        "\n        const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[e] + (int64_t)l * lora_stride_a;",
        "\n        const uint16_t *A = (const uint16_t *)(intptr_t)w_ptr_a[e];"),
    "w2 B transposed": ("d += xa[r] * bf(B[(int64_t)c * rank + r]);",
                        "d += xa[r] * bf(B[(int64_t)r * H + c]);"),
    "w2 y dropped": ("o[c] = bf(yp[c]);", "o[c] = 0.0;"),
    "w2 I loop short": ("for (int32_t i = 0; i < I; ++i)", "for (int32_t i = 0; i < I - 1; ++i)"),
    "workitems keep empty blocks": ("        if (end <= start)\n            continue;",
                                    "        if (end < start)\n            continue;"),
    "workitems rows short": ("item_rows[n_items] = end - start;", "item_rows[n_items] = end - start - 1;"),
    "workitems adapted reversed": ("const int32_t e = (int32_t)adapted[i];",
                                   "const int32_t e = (int32_t)adapted[n_adapted - 1 - i];"),
    "workitems start of next expert": ("const uint32_t start = expert_offsets[e];",
                                       "const uint32_t start = expert_offsets[e + 1];"),
}

RUNNER = r"""
import sys, traceback
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from oracle import oracle as O
import test_oracle_pins as P
failed = []
with O.using({lib!r}):
    for name in sorted(dir(P)):
        if not name.startswith("test_"):
            continue
        fn = getattr(P, name)
        params = getattr(fn, "pytestmark", [])
        argsets = [()]
        for m in params:
            if m.name == "parametrize":
                argsets = [(v,) for v in m.args[1]]
        for args in argsets:
            try:
                fn(*args)
            except Exception:
                failed.append(name)
print("FAILED_PINS", sorted(set(failed)))
"""


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutated = src.replace(old, new, 1)
    d = os.path.join(tmp, name.replace(" ", "_").replace("/", "_"))
    os.makedirs(d)
    c_path, so_path = os.path.join(d, "m.c"), os.path.join(d, "m.so")
    open(c_path, "w").write(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", c_path, "-o", so_path],
                   check=True)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=so_path)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=env)
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED_PINS")]
    assert line, f"runner for {name!r} crashed: {r.stderr[-2000:]}"
    return eval(line[0][len("FAILED_PINS"):])


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            futs = {name: ex.submit(_run_mutant, name, old, new, tmp)
                    for name, (old, new) in MUTANTS.items()}
            results = {name: f.result() for name, f in futs.items()}
    survivors = [n for n, failed in results.items() if not failed]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_unmutated_copy_passes_every_pin():
    with tempfile.TemporaryDirectory() as tmp:
        failed = _run_mutant("identity", "#include <stdint.h>", "#include <stdint.h>", tmp)
    assert failed == []
