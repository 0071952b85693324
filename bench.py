#!/usr/bin/env python3
"""Benchmark of the MI355X fused inference attention forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]
                    [--secondary c1,c3,c4,c5,paged_prefill,mtp_decode,int8_decode,...]

One step is one fia_run (phase 2) of the headline workload: the GQA causal
prefill, bf16, B=4, Q_N=32, KV_N=8, max S=4096, D=128, BSND, per-batch
lengths uniform in [1024, 4096] (seeded).  Inputs are resident in HBM before
the timed region; the plan (phase 1, host validation + schedule upload) is
built once and the C planner call's own time is reported separately
(`phase1_us`), beside the wrapper's time with torch's allocations of the
outputs and workspace.  `value` is algorithmic TFLOP/s: 2 * (D_qk + D_v)
flops per allowed (query, key) pair, pairs counted exactly from the lengths
and the mask mode (masked pairs and skipped tiles are not counted).  The
headline's input tensors (205 MB with padding; the valid rows read are 98 MB)
fit in the 256 MB MALL (Infinity Cache), so repeated runs read them from
there rather than from HBM; each line states its input tensor bytes and
whether they fit, and where they fit it also times single runs with the
inputs evicted first (a 512 MB buffer rewritten before each run).  Beside
the K-step mean, every line gives the median and the minimum of 20 single
runs, each between its own HIP events.

The other workloads (dense causal fp16 prefill, paged GQA decode, varlen TND
prefill, block-sparse prefill, chunked prefill against a paged cache,
multi-token decode against a paged cache, decode against a contiguous and a
paged int8 KV cache, block-sparse prefill with FP8 inputs, MLA decode) are
timed the same way and reported under "secondary"; the decode lines are in
GB/s of algorithmic bytes (every KV byte of every kv head once, plus q, out,
lse, the block-table entries and the dequant scales read).

The JSON line carries the roofline of the headline kernel (achieved from HIP
events on the stream the kernel runs on) and the fp64 CPU oracle timed on a
bounded sample of the same workload on this host (`cpu_baseline`), plus the
oracle on a sample of the paged decode workload in GB/s with all host
threads and with one, and the smallest prefill workload on one thread
(`cpu_baseline_more`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (the FP8 block-sparse inputs' dtype)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def allowed_pairs_fia(case) -> int:
    """Exact number of allowed (i, j) pairs summed over batches and query
    heads (counts only, from lengths and the mask mode)."""
    import numpy as np
    B = case.B
    lq = case.lq if case.lq is not None else np.full(B, case.Sq)
    lkv = case.lkv if case.lkv is not None else np.full(B, case.Skv)
    total = 0
    for b in range(B):
        Lq, Lkv = int(lq[b]), int(lkv[b])
        if case.decode:
            total += Lkv
            continue
        i = np.arange(Lq, dtype=np.int64)
        d = Lkv - Lq
        if case.sparse_mode == 3:
            hi = np.minimum(i + d, Lkv - 1)
            lo = np.zeros_like(i)
        elif case.sparse_mode == 2:
            hi = np.minimum(i, Lkv - 1)
            lo = np.zeros_like(i)
        elif case.sparse_mode == 0 and case.atten_mask is None:
            hi = np.full_like(i, Lkv - 1)
            lo = np.zeros_like(i)
        else:
            raise ValueError("pair count implemented for modes 0 (no mask), 2, 3")
        total += int(np.clip(hi - lo + 1, 0, None).sum())
    return total * case.QN


def allowed_pairs_bsa(case) -> int:
    import numpy as np
    m = case.block_mask.detach().cpu().numpy() != 0
    B, _, nqb, nkb = m.shape
    lq = case.lq if case.lq is not None else np.full(B, case.Sq)
    lkv = case.lkv if case.lkv is not None else np.full(B, case.Skv)
    total = 0
    for b in range(B):
        rows = np.clip(np.minimum((np.arange(nqb) + 1) * case.X, lq[b]) - np.arange(nqb) * case.X, 0, None)
        cols = np.clip(np.minimum((np.arange(nkb) + 1) * case.Y, lkv[b]) - np.arange(nkb) * case.Y, 0, None)
        total += int(np.einsum("hqk,q,k->", m[b].astype(np.int64), rows, cols))
    return total


def decode_bytes(case) -> int:
    import numpy as np
    L = case.lkv.astype(np.int64)
    dv = 0 if case.meta.get("v_is_k") else case.Dv     # value read from the key's bytes
    kv = int(L.sum()) * case.KVN * (case.Dqk + dv) * case.k.element_size()
    if getattr(case, "quant", None):
        # dequant scales/offsets: per channel whole, per token the tokens read
        for key in ("dequant_scale_key", "dequant_offset_key", "dequant_scale_value",
                    "dequant_offset_value"):
            t = case.quant.get(key)
            mode = case.quant["key_quant_mode" if "key" in key else "value_quant_mode"]
            if t is not None:
                kv += t.numel() * t.element_size() if mode == 0 else int(L.sum()) * 4
    rows = case.B * case.QN * case.Sq          # query rows (decode: S = 1)
    qo = rows * (case.Dqk + case.Dv) * 2
    if getattr(case, "rope", None):
        # MLA: the key_rope pool rows read and the query_rope rows
        dr = case.rope["key_rope"].shape[-1]
        kv += int(L.sum()) * dr * 2
        qo += rows * dr * 2
    lse = rows * 4 if case.return_lse else 0
    bt = 4 * int(((L + case.block_size - 1) // case.block_size).sum()) if case.block_table is not None else 0
    return kv + qo + lse + bt


def measured_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it was taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")
    src = os.path.join(ROOT, "attention_fia_fwd_amd", "csrc", "fia_kernels.hip")
    if not os.path.exists(path):
        return None
    kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if kv.get("kernel_source_sha256_prefix") != sha or f"{name}_fetch_kib" not in kv:
        return None
    return int(float(kv[f"{name}_fetch_kib"]) * 1024 * float(kv["fetch_scale"]) +
               float(kv[f"{name}_write_kib"]) * 1024 * float(kv["write_scale"]))


def time_plan(plan, steps: int, warmup: int):
    """Warm up, then time `steps` runs: wall clock between synchronizations
    and HIP events on the stream the kernels are launched on."""
    import torch
    # warm-up: at least `warmup` runs and at least 0.5 s, so clocks settle
    t_end = time.perf_counter() + 0.5
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        plan.run()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        plan.run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = e0.elapsed_time(e1) / 1e3 / steps
    return wall, ev


def sample_launches(plan, n: int = 20, flush=None):
    """Per-launch HIP event times (ms) of `n` single runs, each bracketed by
    its own events on the launch stream after a synchronization; with
    `flush` (a device buffer larger than the 256 MB MALL) the buffer is
    rewritten before each run so the run starts with its inputs evicted.
    Returns (median, min)."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(n):
        if flush is not None:
            flush.add_(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plan.run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return statistics.median(times), min(times)


def build_plan(name, case):
    """Phase 1 on the case, twice: the first plan of a process also pays
    one-time set-up (the code object's load on the device); the second is
    what a caller that re-plans every step pays.  Returns the second plan,
    its C planner call's own time (validation, schedule, the synchronous
    upload of the schedule), the whole wrapper's time (which adds torch's
    allocations of out, lse and workspace) and the first call's C time."""
    from fia_gpu import bsa_plan, fia_plan, to_dev
    to_dev(case)
    make = bsa_plan if name in ("c5", "fp8_bsa") else fia_plan
    first = make(case)
    first_us = first.phase1_s * 1e6
    first.close()
    t0 = time.perf_counter()
    plan = make(case)
    t1 = time.perf_counter()
    return plan, plan.phase1_s * 1e6, (t1 - t0) * 1e6, first_us


DECODE_WORKLOADS = ("c3", "mtp_decode", "int8_decode", "int8_paged_decode", "mla_decode", "mla_shared_kv")
MALL_BYTES = 256 << 20        # MI355X Infinity Cache (MALL)


def input_bytes(case) -> int:
    """Bytes of every input tensor of the run (q, k, v, pools, tables, masks,
    scales; padding rows included), for the statement of what fits in the
    MALL."""
    import torch
    n = 0
    for t in (case.q, case.k, case.v, getattr(case, "atten_mask", None),
              getattr(case, "block_table", None), getattr(case, "block_mask", None)):
        if t is not None:
            n += t.numel() * t.element_size()
    if getattr(case, "meta", {}).get("v_is_k"):
        n -= case.v.numel() * case.v.element_size()
    for extra in ("quant", "fp8", "rope"):
        d = getattr(case, extra, None) or {}
        for t in d.values():
            if isinstance(t, torch.Tensor):
                n += t.numel() * t.element_size()
    return n


def measure(name, steps, warmup):
    import torch
    import workloads as W
    case = W.WORKLOADS[name](device="cuda")
    torch.cuda.synchronize()
    plan, phase1_us, plan_total_us, first_us = build_plan(name, case)
    wall, ev = time_plan(plan, steps, warmup)
    inb = input_bytes(case)
    med, mn = sample_launches(plan)
    res = {"workload": case.name, "steps": steps, "ms_per_step": wall * 1e3,
           "kernel_ms": ev * 1e3, "kernel_ms_median": med, "kernel_ms_min": mn,
           "phase1_us": round(phase1_us, 1),
           "plan_with_allocations_us": round(plan_total_us, 1),
           "phase1_first_in_process_us": round(first_us, 1), "input_tensor_bytes": inb,
           "inputs_fit_mall": inb <= MALL_BYTES}
    if inb <= MALL_BYTES:
        # the same runs with the inputs evicted from the MALL first (a 512 MB
        # buffer rewritten before each run)
        flush = torch.zeros(2 * MALL_BYTES // 4, dtype=torch.int32, device="cuda")
        fmed, fmin = sample_launches(plan, flush=flush)
        del flush
        res.update(kernel_ms_median_mall_flushed=fmed, kernel_ms_min_mall_flushed=fmin)
    if name in DECODE_WORKLOADS:
        nbytes = decode_bytes(case)
        res.update(value=nbytes / wall / 1e9, unit="GB/s", algorithmic_bytes=nbytes,
                   roofline={"bound": "hbm", "achieved": nbytes / ev / 1e9, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": nbytes / ev / 1e9 / PEAK_HBM_GBS})
        if name in ("mla_decode", "mla_shared_kv"):
            # MFMA work beside the bytes: 2 (576 + 512) flops per (query row, kv token)
            flops = 2 * (case.Dqk + case.rope["query_rope"].shape[-1] + case.Dv) * case.QN * int(case.lkv.sum())
            res.update(algorithmic_flops=flops, mfma_tflops=flops / ev / 1e12)
    else:
        if name in ("c5", "fp8_bsa"):
            pairs = allowed_pairs_bsa(case)
            flops = 2 * (case.D + case.D) * pairs
        else:
            pairs = allowed_pairs_fia(case)
            flops = 2 * (case.Dqk + case.Dv) * pairs
        peak = PEAK_FP8_TFLOPS if name == "fp8_bsa" else PEAK_BF16_TFLOPS
        res.update(value=flops / wall / 1e12, unit="TFLOP/s", algorithmic_flops=flops,
                   roofline={"bound": "mfma", "achieved": flops / ev / 1e12,
                             "peak": peak, "unit": "TFLOP/s",
                             "frac": flops / ev / 1e12 / peak})
    res["roofline"]["traffic"] = measured_traffic(name)
    plan.close()
    del case
    torch.cuda.empty_cache()
    return res


def cpu_baseline_decode(name="c3", target_s=8.0, threads=None, case=None):
    """The fp64 oracle on a seeded sample of (batch, head) rows of a decode
    workload; each row is credited with its share of the workload's
    algorithmic bytes (its kv head's cache divided over the G heads that
    share it, plus its q / out / lse bytes and table entries), so the rate is
    in the GB/s of the decode metric."""
    import numpy as np
    import oracle
    import workloads as W
    case = case if case is not None else W.WORKLOADS[name](device="cpu")
    total = decode_bytes(case)
    rows_all = case.B * case.QN
    lkv = case.lkv.astype(np.int64)
    G = case.QN // case.KVN
    per_b = lkv * case.KVN * (case.Dqk + case.Dv) * case.k.element_size()  # cache bytes of batch b
    # share of each row: its batch's cache / QN (= kv head cache / G), rest evenly
    rest = (total - int(per_b.sum())) / rows_all
    rng = np.random.default_rng(98)
    before = oracle.num_threads()
    if threads:
        oracle.set_threads(threads)
    used = oracle.num_threads()
    try:
        def rows_of(n):
            return [(int(rng.integers(case.B)), int(rng.integers(case.QN)), 0) for _ in range(n)]

        def bytes_of(rows):
            return sum(per_b[b] / case.QN + rest for b, _, _ in rows)

        pilot = rows_of(32)
        t0 = time.perf_counter()
        oracle.attention(case, rows=pilot)
        dt = time.perf_counter() - t0
        n = int(min(rows_all * 4, max(32, 32 * target_s / max(dt, 1e-3))))
        rows = rows_of(n)
        t0 = time.perf_counter()
        oracle.attention(case, rows=rows)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_threads(before)
    return {"value": float(bytes_of(rows) / dt / 1e9), "unit": "GB/s", "cores": used, "kind": "oracle",
            "seconds": round(dt, 2), "G": G,
            "sample": f"{n} seeded random (batch, head) rows of {case.name}, fp64, "
                      f"each credited with its share of the algorithmic bytes"}


def cpu_baseline_c1_single_thread():
    """The fp64 oracle on the whole dense causal fp16 workload, one thread."""
    import oracle
    import workloads as W
    case = W.WORKLOADS["c1"](device="cpu")
    before = oracle.num_threads()
    oracle.set_threads(1)
    try:
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 1.0:
            oracle.attention(case)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    finally:
        oracle.set_threads(before)
    flops = 2 * (case.Dqk + case.Dv) * allowed_pairs_fia(case)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "ms_per_run": round(dt * 1e3, 3), "sample": f"the whole of {case.name}, {reps} runs"}


def cpu_baseline(name="c2", target_s=15.0):
    """The fp64 oracle as it is, on a seeded sample of query rows of the
    headline workload, on this host's cores."""
    import numpy as np
    import oracle
    import workloads as W
    case = W.WORKLOADS[name](device="cpu")
    lq = case.lq
    rng = np.random.default_rng(99)

    def rows_of(n):
        out = []
        for _ in range(n):
            b = int(rng.integers(case.B))
            out.append((b, int(rng.integers(case.QN)), int(rng.integers(int(lq[b])))))
        return out

    def flops_of(rows):
        # causal, Lq = Lkv: row i sees i + 1 keys
        return sum(2 * (case.Dqk + case.Dv) * (i + 1) for _, _, i in rows)

    pilot = rows_of(2048)
    t0 = time.perf_counter()
    oracle.attention(case, rows=pilot)
    dt = time.perf_counter() - t0
    n = int(min(5_000_000, max(2048, 2048 * target_s / max(dt, 1e-3))))
    rows = rows_of(n)
    t0 = time.perf_counter()
    oracle.attention(case, rows=rows)
    dt = time.perf_counter() - t0
    fl = flops_of(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{n} seeded random (batch, head, row) query rows of {case.name}, "
                      f"fp64, OpenMP over rows"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2",
                    help="headline workload (c2) or one of: c1, c3, c4, c5, paged_prefill, mtp_decode, "
                         "int8_decode, int8_paged_decode, fp8_bsa, mla_decode, mla_shared_kv")
    ap.add_argument("--secondary", default="c1,c3,c4,c5,paged_prefill,mtp_decode,int8_decode,int8_paged_decode,fp8_bsa,mla_decode,mla_shared_kv",
                    help="comma list of other workloads to time ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the kernels run on a single MI355X and the "
              f"multi-GPU sharding is a design, not code (asked for --gpus {args.gpus}); "
              f"run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}))
        return
    # rebuild when a source is newer than the library, so a stale binary is
    # never measured
    from attention_fia_fwd_amd.build import build
    build(force=False)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)

    head = measure(args.workload, args.steps, args.warmup)
    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        secondary[name] = measure(name, max(5, args.steps // 2), max(2, args.warmup // 2))
        print(f"# {name}: {json.dumps(secondary[name])}", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload if args.workload in ("c2",) else "c2")
    cpu_more = None
    if not args.no_cpu_baseline:
        import workloads as W
        c3 = W.WORKLOADS["c3"](device="cpu")
        cpu_more = {"c3": cpu_baseline_decode("c3", case=c3),
                    "c3_single_thread": cpu_baseline_decode("c3", target_s=4.0, threads=1, case=c3),
                    "c1_single_thread": cpu_baseline_c1_single_thread()}
        print(f"# cpu baselines: {json.dumps(cpu_more)}", file=sys.stderr, flush=True)
    is_decode = args.workload == "c3"
    line = {
        "metric": "prefill TFLOP/s (% bf16 MFMA peak); paged decode KV GB/s (% HBM peak)",
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if args.workload == "c1" else "bf16",
        "data": "synthetic (seeded N(0,1) inputs of the workload's shapes and length mix)",
        "config": {"workload": head["workload"], "kernel_ms": head["kernel_ms"],
                   "kernel_ms_median": head["kernel_ms_median"], "kernel_ms_min": head["kernel_ms_min"],
                   "kernel_ms_median_mall_flushed": head.get("kernel_ms_median_mall_flushed"),
                   "phase1_us": head["phase1_us"],
                   "plan_with_allocations_us": head["plan_with_allocations_us"],
                   "phase1_first_in_process_us": head["phase1_first_in_process_us"],
                   "input_tensor_bytes": head["input_tensor_bytes"],
                   "inputs_resident_in_mall": head["inputs_fit_mall"],
                   "device": getattr(props, "gcnArchName", props.name),
                   "compute_units": props.multi_processor_count},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "cpu_baseline_more": cpu_more,
        "secondary": secondary,
    }
    if is_decode:
        line["config"]["note"] = "decode workload"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
