#!/usr/bin/env python3
"""Benchmark of SGMV expand-slice on one MI355X.

One step = one call of the hot path (sgmv_expand_slice, or one
sgmv_expand_multi_slice call for the fused QKV workload) over one batch of
seeded synthetic input already resident in HBM.  W untimed warm-up steps,
then exactly K timed steps between HIP events on the launch stream, bracketed
by device synchronisation.  Each step uses the next of S identical buffer
sets (inputs, weights, output), S >= 2 and S * footprint >= 1 GiB, so no
step finds its data in the 256 MB Infinity Cache or the L2s.

Effective bandwidth uses the algorithmic byte count
    T_act * rank * in_bytes + sum_distinct_adapters slice * rank * w_bytes
    + T_act * slice * out_bytes * (1 + add_inputs)
(T_act = rows of segments whose adapter index is not -1; summed over slices
for the fused call).  tokens/s counts every row handed to the call once.

Prints ONE JSON line.  Also reports the CPU oracle (bounded sample, host
cores) as a baseline and the HBM traffic measured with rocprofv3 counters
when a summary for the current kernel source is committed under profiles/.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E peak, GB/s
DEFAULT_WORKLOAD = "llama7b_q_proj"
CSRC = os.path.join(ROOT, "segmented_gather_gemm_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


SHARED_SOURCES = ("sgmv_common.h", "sgmv_launch.h", "sgmv_host.h", "sgmv_host.cpp")


def kernel_source_hash(family: str = "expand") -> str:
    """Hash of the library sources a kernel family is built from (kernels,
    launch and entry points): the expand's files are every source not named
    sgmv_shrink*; the shrink's (LoRA-A projection) are the sgmv_shrink* files
    and the shared ones."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        if family == "expand" and name.startswith("sgmv_shrink"):
            continue
        if family == "shrink" and not (name.startswith("sgmv_shrink") or name in SHARED_SOURCES):
            continue
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def byte_model(wl):
    """Algorithmic bytes of one call, active rows, distinct adapters."""
    from sgmv_workloads import DTYPE_BYTES
    act = wl.active_mask()
    t_act = int(wl.lens[act].sum())
    distinct = len(set(wl.idx[act].tolist()))
    total = 0
    ob = DTYPE_BYTES[wl.out_dtype]
    for s in wl.slices:
        total += t_act * wl.K * DTYPE_BYTES[s.x_dtype]
        total += distinct * s.N * wl.K * DTYPE_BYTES[s.w_dtype]
        total += t_act * s.N * ob * (2 if wl.add else 1)
    return total, t_act, distinct


def footprint_bytes(wl):
    """Device bytes one buffer set occupies."""
    n = wl.out0.nbytes
    for s in wl.slices:
        n += s.x.nbytes + s.w.nbytes
    return n


class BufferSet:
    def __init__(self, wl, device):
        import numpy as np
        from sgmv_workloads import to_torch
        self.x = [to_torch(s.x, s.x_dtype, device) for s in wl.slices]
        self.w = [to_torch(np.ascontiguousarray(s.w), s.w_dtype, device) for s in wl.slices]
        self.out = to_torch(wl.out0, wl.out_dtype, device)

    def clone(self):
        c = object.__new__(BufferSet)
        c.x = [t.clone() for t in self.x]
        c.w = [t.clone() for t in self.w]
        c.out = self.out.clone()
        return c


def make_step(wl, meta, sets, split=False):
    """One step: one call over the whole workload (the fused multi-slice call
    for several slices), or with `split` one single-slice call per slice."""
    import segmented_gather_gemm_amd as sg
    start, lens, idx = meta
    B, M = wl.batches, wl.max_seq_len
    if wl.per_token:
        s = wl.slices[0]

        def step(i):
            bs = sets[i % len(sets)]
            sg.bgmv_expand_slice(bs.x[0], bs.w[0], bs.out, idx, s.offset, s.N, wl.add)
    elif len(wl.slices) == 1 or split:
        def step(i):
            bs = sets[i % len(sets)]
            for k, s in enumerate(wl.slices):
                sg.sgmv_expand_slice(bs.x[k], bs.w[k], bs.out, start, lens, idx, B, M, s.offset,
                                     s.N, wl.add)
    else:
        offs = [s.offset for s in wl.slices]

        def step(i):
            bs = sets[i % len(sets)]
            sg.sgmv_expand_multi_slice(list(zip(bs.x, bs.w, offs)), bs.out, start, lens, idx,
                                       B, M, wl.add)
    return step


def time_steps(step, steps, warmup):
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        step(warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / steps, wall


def time_steps_graph(step, steps, warmup, batches=5):
    """Capture `warmup` steps and the `steps` timed steps (as up to `batches`
    consecutive batches) into HIP graphs and replay them back to back: the
    same launches with the host's launch overhead taken out of the loop.
    Returns (ms per step over all timed steps, wall seconds, median over the
    batches of ms per step)."""
    import statistics
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):            # first calls fill the library's device caches
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    nb = max(1, min(batches, steps))
    sizes = [steps // nb + (1 if b < steps % nb else 0) for b in range(nb)]
    g_warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        for i in range(warmup):
            step(i)
    graphs, first = [], warmup
    for n in sizes:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(first + i)
        graphs.append(g)
        first += n
    torch.cuda.synchronize()
    g_warm.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for b, g in enumerate(graphs):
        g.replay()
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_batch = [ev[b].elapsed_time(ev[b + 1]) / sizes[b] for b in range(nb)]
    return ev[0].elapsed_time(ev[nb]) / steps, wall, statistics.median(per_batch)


def time_single_launches(step, reps=50, flush_bytes=1 << 30):
    """Median time of single launches, each right after a write of
    `flush_bytes` that evicts the caches; events bracket the launch only (it
    is enqueued while the flush still runs, so host latency is not timed)."""
    import statistics
    import torch
    flush = torch.empty(flush_bytes // 4, dtype=torch.int32, device="cuda")
    times = []
    for i in range(reps):
        flush.fill_(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    return statistics.median(times)


def copy_ceiling(nbytes, device, reps=20):
    """GB/s of a plain device copy moving `nbytes` read + `nbytes` written
    (context only)."""
    import torch
    n = max(1, nbytes // 2)
    sets = max(2, math.ceil((1 << 30) / (2 * n)))
    src = [torch.empty(n, dtype=torch.int16, device=device).fill_(1) for _ in range(sets)]
    dst = [torch.empty_like(s) for s in src]
    for i in range(5):
        dst[i % sets].copy_(src[i % sets])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(reps):
        dst[i % sets].copy_(src[i % sets])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    return 2 * n * 2 / (ms * 1e-3) / 1e9


def traffic_from_profiles(workload, ksha):
    """Measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a
    plain copy) from a committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M)
    b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not b or m.group(1) != ksha:
        return None
    return float(b.group(1))


def cpu_baseline(wl, model_bytes, budget_s):
    """Time the CPU oracle (as it stands) on the same workload, repeating the
    whole call until about `budget_s` seconds of CPU time have been spent (a
    bounded sample for big workloads: a prefix of the segments), on all host
    cores; then once on one core (a smaller prefix if needed)."""
    import numpy as np
    import oracle
    import sgmv_workloads as W
    threads = len(os.sched_getaffinity(0))
    slices = [oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices]

    def sample_for(seconds, nthreads):
        # estimate: ~1e8 fp64 multiply-adds per second per thread
        work_rows = int(wl.lens[wl.active_mask()].sum())
        macs = work_rows * sum(s.N for s in wl.slices) * wl.K
        if macs / (1e8 * nthreads) <= seconds:
            return wl, "full workload"
        keep = max(1, int(len(wl.lens) * seconds * 1e8 * nthreads / macs))
        idx = wl.idx.copy()
        idx[keep:] = -1
        return (W.Workload(wl.name, wl.slices, wl.out0, wl.out_dtype, wl.start, wl.lens, idx,
                           wl.add, wl.K, wl.L), f"first {keep} of {len(wl.lens)} segments")

    def run(sample, nthreads, seconds, max_reps):
        out = np.empty_like(sample.out0)
        reps, spent = 0, 0.0
        while reps == 0 or (spent < seconds and reps < max_reps):
            out[...] = sample.out0
            t0 = time.perf_counter()
            oracle.expand(slices, out, sample.out_dtype, sample.start, sample.lens, sample.idx,
                          sample.add, sample.K, sample.L, threads=nthreads)
            spent += time.perf_counter() - t0
            reps += 1
        return spent / reps, reps

    sample, note = sample_for(budget_s, threads)
    secs, reps = run(sample, threads, budget_s, 1000)
    sample_bytes, _, _ = byte_model(sample)
    one, one_note = sample_for(budget_s / 4, 1)
    secs1, _ = run(one, 1, 0.0, 1)
    one_bytes, _, _ = byte_model(one)
    return {"value": round(sample_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_call": round(secs, 4), "reps": reps,
            "sample": f"{note} of {wl.name} seed {wl.seed}, fp64 C oracle, {reps} calls",
            "single_core_gbs": round(one_bytes / secs1 / 1e9, 4),
            "single_core_sample": f"{one_note}, one call"}


# ---------------------------------------------------------------------------
# LoRA-A projection (shrink) workloads.
# ---------------------------------------------------------------------------

def shrink_byte_model(wl, rows=None):
    """Algorithmic bytes of one shrink call: the input rows of active
    segments, each distinct adapter's lora_A rows once per slice, and the
    projected rows written.  `rows`: count only these (active) rows."""
    import numpy as np
    from sgmv_workloads import DTYPE_BYTES
    ra = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if a >= 0 and n > 0:
            ra[s:s + n] = a
    act = np.nonzero(ra >= 0)[0] if rows is None else np.asarray(rows)
    t_act = len(act)
    distinct = len(set(ra[act].tolist()))
    ns = len(wl.lora_a)
    total = t_act * wl.H * DTYPE_BYTES[wl.x_dtype]
    total += ns * distinct * wl.K * wl.H * DTYPE_BYTES[wl.a_dtype]
    total += ns * t_act * wl.K * DTYPE_BYTES[wl.out_dtype]
    return total, t_act, distinct


class ShrinkBufferSet:
    def __init__(self, wl, device):
        import numpy as np
        from sgmv_workloads import to_torch
        self.x = to_torch(wl.x, wl.x_dtype, device)
        self.a = [to_torch(np.ascontiguousarray(a).reshape(a.shape[0], -1), wl.a_dtype,
                           device).view(a.shape) for a in wl.lora_a]
        self.outs = [to_torch(o, wl.out_dtype, device) for o in wl.outs0]

    def clone(self):
        c = object.__new__(ShrinkBufferSet)
        c.x = self.x.clone()
        c.a = [t.clone() for t in self.a]
        c.outs = [t.clone() for t in self.outs]
        return c


def make_shrink_step(wl, meta, sets, split=False):
    """One step: one sgmv_shrink_multi_slice call over every slice (with
    `split`, one sgmv_shrink call per slice)."""
    import segmented_gather_gemm_amd as sg
    start, lens, idx = meta
    B, M = wl.batches, wl.max_seq_len

    if split:
        def step(i):
            bs = sets[i % len(sets)]
            for a, o in zip(bs.a, bs.outs):
                sg.sgmv_shrink(bs.x, a, o, start, lens, idx, B, M, wl.scale)
    else:
        def step(i):
            bs = sets[i % len(sets)]
            sg.sgmv_shrink_multi_slice(bs.x, list(zip(bs.a, bs.outs)), start, lens, idx, B, M,
                                       wl.scale)
    return step


def shrink_cpu_baseline(wl, budget_s):
    """Time the CPU oracle's shrink (as it stands) on a bounded sample of the
    workload: the first active rows, as many as about `budget_s` seconds of
    work on all host cores allow; then a smaller sample on one core."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    ra = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if a >= 0 and n > 0:
            ra[s:s + n] = a
    active = np.nonzero(ra >= 0)[0]
    macs_per_row = wl.H * wl.K * len(wl.lora_a)

    def sample_for(seconds, nthreads):
        # estimate: ~2e8 fp64 multiply-adds per second per thread
        keep = int(seconds * 2e8 * nthreads / macs_per_row)
        keep = max(1, min(len(active), keep))
        note = "all active rows" if keep == len(active) else f"first {keep} of {len(active)} active rows"
        return active[:keep], note

    def run(rows, nthreads, seconds, max_reps):
        reps, spent = 0, 0.0
        while reps == 0 or (spent < seconds and reps < max_reps):
            outs = [o.copy() for o in wl.outs0]
            t0 = time.perf_counter()
            oracle.shrink(wl.x, wl.x_dtype, wl.lora_a, wl.a_dtype, outs, wl.out_dtype, wl.start,
                          wl.lens, wl.idx, wl.scale, rows=rows, threads=nthreads)
            spent += time.perf_counter() - t0
            reps += 1
        return spent / reps, reps

    rows, note = sample_for(budget_s, threads)
    secs, reps = run(rows, threads, budget_s, 1000)
    sample_bytes, _, _ = shrink_byte_model(wl, rows)
    rows1, note1 = sample_for(budget_s / 4, 1)
    secs1, _ = run(rows1, 1, 0.0, 1)
    one_bytes, _, _ = shrink_byte_model(wl, rows1)
    return {"value": round(sample_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_call": round(secs, 4), "reps": reps,
            "sample": f"{note} of {wl.name} seed {wl.seed}, fp64 C oracle, {reps} calls",
            "single_core_gbs": round(one_bytes / secs1 / 1e9, 4),
            "single_core_sample": f"{note1}, one call"}


def run_shrink(args):
    import math as _m
    import torch
    import sgmv_workloads as W
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    log(f"bench: generating {args.workload} seed {args.seed}")
    wl = W.SHRINK_WORKLOADS[args.workload](args.seed)
    model_bytes, t_act, distinct = shrink_byte_model(wl)
    fp = wl.x.nbytes + sum(a.nbytes for a in wl.lora_a) + sum(o.nbytes for o in wl.outs0)
    nsets = max(2, _m.ceil((1 << 30) / fp))
    log(f"bench: {len(wl.lora_a)} slice(s), T={wl.T} (active {t_act}), hidden {wl.H} -> rank "
        f"{wl.K}, {distinct} distinct adapters, {model_bytes / 1e6:.2f} MB per call, {nsets} "
        f"rotated buffer sets of {fp / 1e6:.1f} MB")
    meta = tuple(torch.from_numpy(a).to(device) for a in (wl.start, wl.lens, wl.idx))
    first = ShrinkBufferSet(wl, device)
    sets = [first] + [first.clone() for _ in range(nsets - 1)]
    torch.cuda.synchronize()
    split = args.split_slices and len(wl.lora_a) > 1
    step = make_shrink_step(wl, meta, sets, split)

    log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (eager launches)")
    ms_eager, wall_eager = time_steps(step, args.steps, args.warmup)
    log(f"bench: eager {ms_eager * 1e3:.2f} us per step")
    ms_median = None
    if args.eager:
        ms, wall, mode = ms_eager, wall_eager, "eager"
    else:
        log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (HIP-graph replay)")
        ms, wall, ms_median = time_steps_graph(step, args.steps, args.warmup)
        mode = "hip-graph replay"
    log("bench: single launches after a cache flush")
    ms_single = time_single_launches(step)
    sec = ms * 1e-3
    gbs = model_bytes / sec / 1e9
    tokens_s = wl.T / sec
    ksha = kernel_source_hash("shrink")
    traffic_bytes = None if split else traffic_from_profiles(args.workload, ksha)
    traffic = None if traffic_bytes is None else round(traffic_bytes / sec / 1e9, 2)
    log(f"bench: {ms * 1e3:.2f} us per step, {gbs:.1f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% "
        f"of peak), {tokens_s / 1e6:.2f} M tokens/s (wall {wall:.2f} s)")
    ceiling = None if args.no_copy_ceiling else round(copy_ceiling(model_bytes // 2, device), 1)
    del sets, first
    torch.cuda.empty_cache()
    cpu = None
    if args.cpu_budget > 0:
        log("bench: timing the CPU oracle baseline")
        cpu = shrink_cpu_baseline(wl, args.cpu_budget)
    result = {
        "metric": "effective HBM GB/s (% of MI355X peak) and tokens/s for sgmv_shrink",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.a_dtype,
        "data": "synthetic",
        "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(tokens_s, 1),
        "config": {
            "workload": args.workload,
            "seed": args.seed,
            "hidden": wl.H,
            "rank": wl.K,
            "slices": len(wl.lora_a),
            "batches": wl.batches,
            "total_tokens": wl.T,
            "active_tokens": t_act,
            "distinct_adapters": distinct,
            "scale": wl.scale,
            "dtypes": {"inputs": wl.x_dtype, "lora_a": wl.a_dtype, "output": wl.out_dtype,
                       "accumulate": "f32"},
            "bytes_per_step": model_bytes,
            "rotated_buffer_sets": nsets,
            "call": (f"{len(wl.lora_a)} x sgmv_shrink" if split else
                     "sgmv_shrink_multi_slice"),
            "launch": mode,
            "batch_median_us_per_step": None if ms_median is None else round(ms_median * 1e3, 3),
            "eager_us_per_step": round(ms_eager * 1e3, 3),
            "single_launch_after_flush_us": round(ms_single * 1e3, 3),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_bytes_per_launch": traffic_bytes,
            # the library runs split-T from 64 units of 64 tokens up, split-H below
            "kernel": "shrink_split_t" if -(-wl.T // 64) >= 64 else "shrink_split_h",
            "kernel_source_sha256_16": ksha,
        },
        "copy_ceiling_gbs": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of CPU-oracle time for the baseline (0 = skip)")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (default: HIP-graph replay, eager also reported)")
    ap.add_argument("--split-slices", action="store_true",
                    help="multi-slice workloads: one single-slice call per slice per step "
                         "instead of one fused multi-slice call")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sgmv_workloads as W
    import segmented_gather_gemm_amd  # noqa: F401  (fails loudly if libsgmv.so is missing)

    if args.workload in W.SHRINK_WORKLOADS:
        return run_shrink(args)
    if args.workload not in W.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from "
                 f"{sorted(W.WORKLOADS) + sorted(W.SHRINK_WORKLOADS)}")
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    log(f"bench: generating {args.workload} seed {args.seed}")
    wl = W.WORKLOADS[args.workload](args.seed)
    model_bytes, t_act, distinct = byte_model(wl)
    fp = footprint_bytes(wl)
    nsets = max(2, math.ceil((1 << 30) / fp))
    log(f"bench: {len(wl.slices)} slice(s), T={wl.T} (active {t_act}), rank {wl.K}, "
        f"{distinct} distinct adapters, {model_bytes / 1e6:.2f} MB per call, "
        f"{nsets} rotated buffer sets of {fp / 1e6:.1f} MB")
    meta = tuple(torch.from_numpy(a).to(device) for a in (wl.start, wl.lens, wl.idx))
    first = BufferSet(wl, device)
    sets = [first] + [first.clone() for _ in range(nsets - 1)]
    torch.cuda.synchronize()
    split = args.split_slices and len(wl.slices) > 1
    step = make_step(wl, meta, sets, split)

    log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (eager launches)")
    ms_eager, wall_eager = time_steps(step, args.steps, args.warmup)
    log(f"bench: eager {ms_eager * 1e3:.2f} us per step")
    ms_median = None
    if args.eager:
        ms, wall, mode = ms_eager, wall_eager, "eager"
    else:
        log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (HIP-graph replay)")
        ms, wall, ms_median = time_steps_graph(step, args.steps, args.warmup)
        mode = "hip-graph replay"
    log("bench: single launches after a cache flush")
    ms_single = time_single_launches(step)
    sec = ms * 1e-3
    gbs = model_bytes / sec / 1e9
    tokens_s = wl.T / sec
    ksha = kernel_source_hash()
    traffic_bytes = None if split else traffic_from_profiles(args.workload, ksha)
    traffic = None if traffic_bytes is None else round(traffic_bytes / sec / 1e9, 2)
    log(f"bench: {ms * 1e3:.2f} us per step, {gbs:.1f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% "
        f"of peak), {tokens_s / 1e6:.2f} M tokens/s (wall {wall:.2f} s)")

    ceiling = None if args.no_copy_ceiling else round(copy_ceiling(model_bytes // 2, device), 1)
    del sets, first
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_budget > 0:
        log("bench: timing the CPU oracle baseline")
        cpu = cpu_baseline(wl, model_bytes, args.cpu_budget)

    dtype = {"f16": "f16", "bf16": "bf16"}[wl.slices[0].w_dtype]
    result = {
        "metric": "effective HBM GB/s (% of MI355X peak) and tokens/s for sgmv_expand_slice",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(tokens_s, 1),
        "config": {
            "workload": args.workload,
            "seed": args.seed,
            "slices": [[s.offset, s.N] for s in wl.slices],
            "rank": wl.K,
            "batches": wl.batches,
            "total_tokens": wl.T,
            "active_tokens": t_act,
            "distinct_adapters": distinct,
            "add_inputs": wl.add,
            "dtypes": {"inputs": wl.slices[0].x_dtype, "lora_b": wl.slices[0].w_dtype,
                       "output": wl.out_dtype, "accumulate": "f32"},
            "bytes_per_step": model_bytes,
            "rotated_buffer_sets": nsets,
            "call": ("sgmv_bgmv_expand_slice" if wl.per_token else
                     "sgmv_expand_slice" if len(wl.slices) == 1 else
                     f"{len(wl.slices)} x sgmv_expand_slice" if split else "sgmv_expand_multi_slice"),
            "launch": mode,
            "batch_median_us_per_step": None if ms_median is None else round(ms_median * 1e3, 3),
            "eager_us_per_step": round(ms_eager * 1e3, 3),
            "single_launch_after_flush_us": round(ms_single * 1e3, 3),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_bytes_per_launch": traffic_bytes,
            "kernel": "expand_fast",
            "kernel_source_sha256_16": ksha,
        },
        "copy_ceiling_gbs": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
