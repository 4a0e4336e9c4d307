#!/usr/bin/env python3
"""Benchmark of the routed LoRA delta on one MI355X.

Workload: decode BGMV at the Llama-3-8B QKV shape (256 one-token rows,
k_in 4096, fused output slices 4096/1024/1024, 32 adapters at max rank 16 with
true ranks in {8, 16}, Zipf(1) routing, 5% unadapted rows, scale 32/r).

A step is one pass of the hot path over one batch: lora_delta_fused_build,
which builds the routing metadata (rows sorted by slot, segments, tile
records; written out for later layers) and applies the fused delta (shrink +
expand, MFMA for segments of at least 16 rows, vector ALU below) in one
launch at this size.  Inputs are resident in HBM and rotate over enough
independent copies (> 1 GiB in total) that no step finds its adapters in the
256 MB Infinity Cache.

Timed region: exactly K steps, replayed from one HIP graph, bracketed by
torch.cuda.synchronize().  value = algorithmic bytes of the K steps / wall
time (GB/s).  The step kernel's average duration is measured with two HIP
events on the launch stream bracketing the replay of a graph of K launches
(elapsed / K; a graph, so that the host's launch rate cannot set the pace);
it gives the roofline fraction against 8 TB/s.  Timed the same way and
reported beside it: the same work in two launches (lora_meta_build, then
lora_delta_fused), each of those kernels alone, and a plain device copy
moving the same number of bytes (plain_copy_same_bytes: what the memory
system gives a transfer of this size).  The fp64 CPU oracle is timed on the
same batch on the host cores (cpu_baseline).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --calibrate-copy   # a plain 512 MiB device copy, for counter scaling
    python bench.py --workload prefill|no_reuse|moe|moe_shared|w2|w2_reuse [--steps K]

The other workloads (prefill SGMV, one adapter per row, MoE gemm1 regular and
shared-A, MoE w2 with and without gemm1's routing) print a secondary line of
the same form: the median of K single calls, each after a 1 GiB write that
evicts the Infinity Cache and the L2s, timed by HIP events on the launch
stream; the fp64 oracle timed on a bounded sample of the same inputs
(cpu_baseline, scaled to GB/s over the workload's algorithmic bytes per row
or pair).

HBM traffic of a workload's main kernel (roofline.traffic) comes from
rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
profiles/<kernel>_<workload>_traffic.txt, scaled by what the same counters read for a
plain copy; it is reported only while the kernel sources still hash to the
recorded value, else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "effective HBM GB/s and tokens/sec of routed LoRA delta (% of peak), 1 MI355X"


KERNEL_DIR = os.path.join(ROOT, "tenant_lora_serving_amd", "csrc")


def kernel_source_hash() -> str:
    """Hash of every kernel source file (so recorded counters match the code)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(KERNEL_DIR)):
        with open(os.path.join(KERNEL_DIR, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch of the workload's main kernel from the recorded
    counter runs (profiles/<kernel>_<workload>_traffic.txt), or None when missing or
    taken on other kernel sources."""
    tag = "fused" if workload in ("decode", "prefill", "no_reuse") else "segment"
    path = os.path.join(ROOT, "profiles", f"{tag}_{workload}_traffic.txt")
    try:
        kv = dict(ln.strip().split("=", 1) for ln in open(path) if "=" in ln and not ln.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256_16") != kernel_source_hash():
        return None
    return {"bytes": int(float(kv["hbm_bytes_per_launch"])), "kernel": kv.get("kernel")}


def calibrate_copy():
    import torch
    torch.cuda.set_device(0)
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "reps": 3}), flush=True)


def algorithmic_bytes(case) -> int:
    """x rows + each active adapter's A and B once + y read and written, all at
    the padded rank (bytes the method must move)."""
    import numpy as np
    act = (case.slot >= 0) & (case.slot < case.num_slots)
    n_act = int(act.sum())
    n_slots_act = len(np.unique(case.slot[act]))
    per_slot = (case.num_slices * case.max_rank * case.k_in + case.n_out * case.max_rank) * 2
    return n_act * case.k_in * 2 + n_slots_act * per_slot + n_act * case.n_out * 4


def cpu_baseline(case, bytes_per_step: int, min_s: float, max_s: float) -> dict:
    import numpy as np
    from oracle import oracle as O
    rows = np.arange(case.n)
    passes, t0 = 0, time.perf_counter()
    while True:
        O.case_fused_rows(case, rows)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_s or el >= max_s:
            break
    return {"value": round(bytes_per_step * passes / el / 1e9, 4), "unit": "GB/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": f"the full {case.n}-row decode batch, fp64 fused delta, {passes} passes in {el:.1f} s"}


def moe_bytes(topk_ids, lora_ids, L, E, a_elems, b_elems, x_row, out_row, out_all_pairs):
    """Activations of adapted tokens or pairs, each touched (adapter, expert)
    pair's weights once, and the output rows (every pair for gemm1, which
    writes zero rows; read and written for the routed pairs of w2)."""
    import numpy as np
    T, top_k = topk_ids.shape
    lo = np.repeat(lora_ids, top_k)
    ex = topk_ids.reshape(-1)
    valid = (lo >= 0) & (lo < L) & (ex >= 0) & (ex < E)
    keys = np.unique(lo[valid] * E + ex[valid])
    w = len(keys) * (a_elems + b_elems) * 2
    if out_all_pairs:  # gemm1: x per adapted token, out for every pair
        t_act = int(((lora_ids >= 0) & (lora_ids < L)).sum())
        return t_act * x_row + w + T * top_k * out_row
    return int(valid.sum()) * (x_row + out_row) + w


def oracle_rate(bytes_per_unit: float, fn, units_per_pass: int, min_s: float, max_s: float, what: str) -> dict:
    """The fp64 oracle timed on a bounded sample (fn computes units_per_pass
    rows or pairs), scaled to GB/s over the workload's algorithmic bytes per
    row or pair."""
    from oracle import oracle as O
    passes, t0 = 0, time.perf_counter()
    while True:
        fn()
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_s or el >= max_s:
            break
    return {"value": round(bytes_per_unit * units_per_pass * passes / el / 1e9, 4), "unit": "GB/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{what}: {units_per_pass} of them per pass, {passes} passes in {el:.1f} s, "
                      "rate scaled by the workload's algorithmic bytes per unit"}


def secondary(args):
    """One of the non-headline workloads: median of single calls, each after a
    1 GiB write that evicts the Infinity Cache and the L2s (cold), timed by
    HIP events on the launch stream; the oracle on a bounded sample of the
    same inputs; HBM traffic of the call's main kernel from recorded counters."""
    import numpy as np
    import torch

    from oracle import oracle as O
    from tenant_lora_serving_amd import inputs as I
    from tenant_lora_serving_amd import lora as B

    torch.cuda.set_device(0)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    w = args.workload
    if w in ("prefill", "no_reuse"):
        case = I.prefill_sgmv() if w == "prefill" else I.no_reuse()
        nbytes = algorithmic_bytes(case)
        rows = case.n
        meta = B.lora_meta_build(torch.from_numpy(case.slot).cuda(), case.num_slots)
        ws = B.fused_workspace(case.n, case.num_slots, case.num_slices, case.max_rank, case.k_in)
        sc = torch.from_numpy(case.scale).cuda()
        x, a, b, y = d16(case.x), d16(case.a_pool), d16(case.b_pool), d16(case.y)
        call = lambda: B.lora_delta_fused(x, a, b, sc, case.slice_sizes, meta, y, ws=ws)  # noqa: E731
        kernel = "fused_kernel (shrink + expand in one launch)"
        desc = {"workload": case.name, "rows": case.n, "k_in": case.k_in, "slices": list(case.slice_sizes),
                "num_slots": case.num_slots, "max_rank": case.max_rank,
                "note": "metadata built once, outside the timed calls"}
        act = np.flatnonzero((case.slot >= 0) & (case.slot < case.num_slots))
        sample = act[:: max(1, len(act) // 64)][:64]
        cpu = lambda: oracle_rate(nbytes / rows, lambda: O.case_fused_rows(case, sample), len(sample),  # noqa
                                  args.cpu_seconds, 30.0, "rows of the batch (fused delta, fp64)")
    elif w in ("moe", "moe_shared"):
        c = I.moe_gemm1()
        E, L, R, H, I_ = c.E, c.L, c.R, c.H, c.I
        shared = w == "moe_shared"
        if shared:
            mats = [d16(c.a_shared), d16(c.b_fused)]
            (ta, sa), (tb, sb) = B.fill_w_ptr(mats[0]), B.fill_w_ptr(mats[1])
            a_el, b_el = R * H, 2 * I_ * R
        else:
            mats = [d16(m) for m in (c.a_gate, c.a_up, c.b_gate, c.b_up)]
            (ta, sa), (tb, sb) = B.fill_w_ptr(mats[0], mats[1]), B.fill_w_ptr(mats[2], mats[3])
            a_el, b_el = 2 * R * H, 2 * I_ * R
        nbytes = moe_bytes(c.topk_ids, c.lora_ids, L, E, a_el, b_el, H * 2, 2 * I_ * 2, True)
        rows = c.T
        x, tk, lo = d16(c.x), torch.from_numpy(c.topk_ids).cuda(), torch.from_numpy(c.lora_ids).cuda()
        ws = B.moe_workspace(c.T, c.top_k, E, L, R, H)
        out = torch.empty((c.T, c.top_k, 2 * I_), dtype=torch.bfloat16, device="cuda")
        call = lambda: B.moe_lora_gemm1_delta(x, ta, sa, tb, sb, tk, lo, R, I_, num_loras=L,  # noqa: E731
                                              scale=c.scale, out=out, ws=ws)
        kernel = "meta_kernel + meta_assemble_kernel (pair metadata) + segment_kernel"
        desc = {"workload": c.name + (" shared-A" if shared else " regular"), "tokens": c.T,
                "pairs": c.T * c.top_k, "note": "one call builds the pair metadata and applies the delta"}
        pairs = np.arange(0, c.T * c.top_k, 8)[:1024]
        cpu = lambda: oracle_rate(nbytes / (c.T * c.top_k), lambda: O.case_moe_pairs(c, shared, pairs),  # noqa
                                  len(pairs), args.cpu_seconds, 30.0, "(token, slot) pairs (gemm1 delta, fp64)")
    elif w in ("w2", "w2_reuse"):
        c = I.moe_w2()
        E, L, R, H, I_ = c.E, c.L, c.R, c.H, c.I
        mats = [d16(c.a_down), d16(c.b_down)]
        (ta, sa), (tb, sb) = B.fill_w_ptr(mats[0]), B.fill_w_ptr(mats[1])
        nbytes = moe_bytes(c.topk_ids, c.lora_ids, L, E, R * I_, H * R, I_ * 2, H * 4, False)
        rows = c.T
        x2, y = d16(c.x2), d16(c.y)
        tk, lo = torch.from_numpy(c.topk_ids).cuda(), torch.from_numpy(c.lora_ids).cuda()
        wt = torch.from_numpy(c.topk_weights).cuda()
        ws = B.moe_w2_workspace(c.T, c.top_k, E, L, R, I_)
        reuse = w == "w2_reuse"
        if reuse:  # the routing of an earlier call on this workspace stands in for gemm1's
            B.moe_lora_w2_delta(x2, ta, sa, tb, sb, tk, lo, R, y, num_loras=L, topk_weights=wt, ws=ws)
        call = lambda: B.moe_lora_w2_delta(x2, ta, sa, tb, sb, tk, lo, R, y, num_loras=L,  # noqa: E731
                                           topk_weights=wt, scale=c.scale, ws=ws, reuse_routing=reuse)
        kernel = "segment_kernel" if reuse else "meta_kernel + meta_assemble_kernel + segment_kernel"
        desc = {"workload": c.name + (" reusing gemm1's routing" if reuse else ""), "tokens": c.T,
                "pairs": c.T * c.top_k}
        lo_p = np.repeat(c.lora_ids, c.top_k)
        valid = np.flatnonzero((lo_p >= 0) & (lo_p < L))
        pairs = valid[:: max(1, len(valid) // 1024)][:1024]
        cpu = lambda: oracle_rate(nbytes / len(valid), lambda: O.case_moe_w2_pairs(c, pairs, True),  # noqa
                                  len(pairs), args.cpu_seconds, 30.0, "routed pairs (w2 delta, fp64)")
    else:
        raise SystemExit(f"unknown workload {w!r}")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    times = []
    for i in range(K):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    ms = float(np.median(times))
    gbs = nbytes / (ms * 1e-3) / 1e9
    desc.update({"bytes_per_call": int(nbytes), "mfma_min_rows": B.mfma_min_rows(),
                 "kernel_sources": kernel_source_hash(), "timing": "median of single cold calls"})
    traffic = recorded_traffic(w)
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded)", "secondary": True,
        "config": desc, "tokens_per_s": round(rows / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_kernel": traffic["kernel"] if traffic else None,
                     "kernel": kernel, "call_us": round(ms * 1e3, 3)}}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu()
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--copies", type=int, default=0, help="independent input copies (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "no_reuse", "moe", "moe_shared", "w2", "w2_reuse"])
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the routed LoRA delta on a single "
              "MI355X (no multi-GPU path); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload != "decode":
        secondary(args)
        return

    import numpy as np
    import torch

    from tenant_lora_serving_amd import inputs as I
    from tenant_lora_serving_amd import lora as B

    torch.cuda.set_device(0)
    case = I.decode_bgmv()
    bytes_step = algorithmic_bytes(case)
    act = (case.slot >= 0) & (case.slot < case.num_slots)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    footprint = case.a_pool.nbytes + case.b_pool.nbytes + case.x.nbytes + case.y.nbytes
    copies = args.copies or max(2, math.ceil((1 << 30) / footprint))
    sets = []
    base = dict(x=d16(case.x), a=d16(case.a_pool), b=d16(case.b_pool), y=d16(case.y),
                scale=torch.from_numpy(case.scale).cuda(), slot=torch.from_numpy(case.slot).cuda())
    # the data rotates over independent copies; the metadata buffers and the
    # workspace are one set reused by every step, as a serving loop reuses them
    meta = B.LoraMeta.allocate(case.n, case.num_slots)
    ws = B.fused_build_workspace(case.n, case.num_slots, case.num_slices, case.max_rank, case.k_in)
    for _ in range(copies):
        s = {k: v.clone() for k, v in base.items()}
        s["meta"] = meta
        s["ws"] = ws
        sets.append(s)
    del base

    def step(s):
        # the routing metadata (written to meta for later layers) and the
        # fused delta: one launch at this size
        B.lora_delta_fused_build(s["x"], s["a"], s["b"], s["scale"], case.slice_sizes, s["slot"], s["y"],
                                 meta=s["meta"], ws=s["ws"])

    def meta_step(s):
        B.lora_meta_build(s["slot"], case.num_slots, s["meta"])

    def delta_step(s):
        B.lora_delta_fused(s["x"], s["a"], s["b"], s["scale"], case.slice_sizes, s["meta"], s["y"], ws=s["ws"])

    for i in range(args.warmup):
        step(sets[i % copies])
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps from one graph
    K = args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step(sets[i % copies])
    g.replay()                       # warm replay (graph upload)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K

    # ---- kernel durations: HIP events on the launch stream bracketing K
    # back-to-back launches, replayed from a graph so that the host's launch
    # rate cannot set the pace
    stream = torch.cuda.current_stream()

    def region(launch, items):
        for i in range(3):
            launch(items[i % len(items)])
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(K):
                launch(items[i % len(items)])
        gr.replay()  # graph upload
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del gr
        return e0.elapsed_time(e1) / K

    build_ms = region(step, sets)
    # the same work in two launches (metadata kernel, then the fused kernel
    # reading the records it wrote), and each of the two alone
    two_ms = region(lambda s_: (meta_step(s_), delta_step(s_)), sets)
    meta_step(sets[0])
    torch.cuda.synchronize()
    delta_ms = region(delta_step, sets)
    meta_ms = region(meta_step, sets)
    # what a plain device copy moving the same bytes (half read, half written)
    # takes when timed the same way, rotating over as many buffers
    half = bytes_step // 2
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda").fill_(1),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(copies)]
    copy_ms = region(lambda c_: c_[1].copy_(c_[0]), bufs)
    del bufs

    value = bytes_step * K / wall / 1e9
    build_gbs = bytes_step / (build_ms * 1e-3) / 1e9
    traffic = recorded_traffic("decode")
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Zipf routing, random bf16 adapters and activations)",
        "config": {"workload": "decode BGMV, Llama-3-8B QKV shape", "rows": case.n,
                   "k_in": case.k_in, "slices": list(case.slice_sizes), "num_slots": case.num_slots,
                   "max_rank": case.max_rank, "active_rows": int(act.sum()),
                   "active_slots": int(len(np.unique(case.slot[act]))),
                   "bytes_per_step": bytes_step, "input_copies": copies,
                   "step": "lora_delta_fused_build: metadata build + fused delta in one launch",
                   "mfma_min_rows": B.mfma_min_rows(), "kernel_sources": kernel_source_hash()},
        "tokens_per_s": round(case.n * K / wall, 1),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(build_gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(build_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic["bytes"] if traffic else None,
                     "kernel": "fused_kernel<3, 1, 0, BuildOp<DenseOpR<16>>> (metadata + delta, one launch)",
                     "kernel_us": round(build_ms * 1e3, 3)},
        "two_launch_step_us": round(two_ms * 1e3, 3),
        "delta_kernel_us": round(delta_ms * 1e3, 3),
        "delta_kernel_frac": round(bytes_step / (delta_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "meta_kernel_us": round(meta_ms * 1e3, 3),
        "plain_copy_same_bytes": {"us": round(copy_ms * 1e3, 3),
                                  "GB/s": round(2 * half / (copy_ms * 1e-3) / 1e9, 2),
                                  "note": "device copy of half the step's bytes (read + write = the step's "
                                          "bytes), K copies replayed from a graph bracketed by events, "
                                          "buffers rotated"},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(case, bytes_step, args.cpu_seconds, 30.0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
