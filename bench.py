#!/usr/bin/env python3
"""Benchmark of SGMV expand-slice on one MI355X.

One step = one call of the hot path (sgmv_expand_slice, or one
sgmv_expand_multi_slice call for the fused QKV workload) over one batch of
seeded synthetic input already resident in HBM.  The default workload is the
largest configuration, the 14336-wide MLP gate/up slice (mlp_gate_up);
--workload selects another.  W untimed warm-up steps, then exactly K timed
steps, captured in one HIP graph and replayed once between HIP events on the
launch stream right behind the W warm-up steps (themselves one graph,
preceded by a cache-evicting fill), bracketed by device synchronisation, so
the timed steps start on a busy GPU and the host's submission is not
timed; this is done five times, after an untimed spin-up of about 50 ms
of replays (the first replays of a process run 10-25% slower while the GPU
leaves its idle state), and the median replay is reported, every replay
listed in the JSON line.  Each step uses the next of S identical buffer sets
(inputs, weights, output), S >= 2 and S * footprint >= 1 GiB, so no step
finds its data in the 256 MB Infinity Cache or the L2s.

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
DEFAULT_WORKLOAD = "mlp_gate_up"
CSRC = os.path.join(ROOT, "segmented_gather_gemm_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Library sources by kernel family (the profiles under profiles/ name the
# hash of the family they measured); the shared ones belong to every family.
SHARED_SOURCES = ("sgmv_common.h", "sgmv_launch.h", "sgmv_host.h", "sgmv_host.cpp",
                  "sgmv_limits.h")
FAMILY_SOURCES = {
    "expand": ("sgmv_api.cpp", "sgmv_device.h", "sgmv_fast_ks", "sgmv_generic.hip", "sgmv_valu"),
    "shrink": ("sgmv_shrink",),
    "fused": ("sgmv_fused", "sgmv_shrink.h", "sgmv_shrink_launch.h", "sgmv_device.h"),
}


def kernel_source_hash(family: str = "expand") -> str:
    """Hash of the library sources a kernel family is built from (kernels,
    launch and entry points, and the shared helpers)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        if name not in SHARED_SOURCES and not name.startswith(FAMILY_SOURCES[family]):
            continue
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


MAX_ROTATED_SETS = 4096


def rotated_sets(footprint):
    """Buffer sets to rotate so that consecutive steps touch >= 1 GiB of
    distinct memory (none finds its data in the 256 MB Infinity Cache or the
    L2s): max(2, ceil(1 GiB / footprint)), at most MAX_ROTATED_SETS -- a
    workload of a few kilobytes (the two-sequence worked example) stays
    cache-resident whatever the rotation, and is measured as launch
    latency."""
    return min(MAX_ROTATED_SETS, max(2, math.ceil((1 << 30) / max(1, footprint))))


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


def _graph_upload(graph, stream):
    """Upload an instantiated graph to the device ahead of its first launch
    (hipGraphUpload through the HIP runtime torch uses), so the first replay
    does not carry it.  Best effort: False if the runtime call is not there."""
    import ctypes
    try:
        path = next(l.split()[-1] for l in open("/proc/self/maps")
                    if "libamdhip64" in l and l.split()[-1].startswith("/"))
        hip = ctypes.CDLL(path)
        return hip.hipGraphUpload(ctypes.c_void_p(graph.raw_cuda_graph_exec()),
                                  ctypes.c_void_p(stream.cuda_stream)) == 0
    except Exception:
        return False


class _Flush:
    """A 1 GiB device buffer; fill() enqueues two writes of it (about half a
    millisecond of GPU work that also evicts the caches)."""

    def __init__(self):
        import torch
        self.buf = torch.empty((1 << 30) // 4, dtype=torch.int32, device="cuda")
        self.n = 0

    def fill(self):
        self.n += 1
        self.buf.fill_(self.n)
        self.buf.fill_(-self.n)


def time_steps_graph(step, steps, warmup, repeats=5):
    """The `warmup` untimed steps and exactly `steps` timed steps as two HIP
    graphs, captured and uploaded ahead; an untimed spin-up (below); then,
    `repeats` times, on the launch stream: a cache-evicting fill, the warm-up
    graph, an event, the timed graph and an event -- so each timed replay
    follows real work (the GPU is neither idle nor waiting for the host when
    it starts) and covers exactly `steps` steps.  The result is the median
    replay.  Returns (median ms per step, wall seconds of the first replay,
    [ms per step of every replay]); the spin-up's replay count and GPU time
    are left in time_steps_graph.spin_up."""
    import statistics
    import torch
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    g_warm = None
    if warmup > 0:
        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm):
            for i in range(warmup):
                step(i)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(warmup + i)
    torch.cuda.synchronize()
    for gr in (g_warm, g):
        if gr is not None:
            _graph_upload(gr, stream)
    flush = _Flush()
    torch.cuda.synchronize()

    # Spin-up, untimed: the first replays after a process starts run 10-25%
    # slower on MI355X (measured: 124, 128, 114, 110 us per step for the
    # first four 20-step replays of the gate/up workload, then 105-107
    # whatever the flush or the warm-up length) while the GPU leaves its idle
    # state, and a median of five short replays does not hide that.  So the
    # timed graph first replays untimed for about 50 ms of GPU time.
    spin = {"replays": 0, "gpu_ms": 0.0}
    while spin["replays"] < 2 or (spin["gpu_ms"] < 50.0 and spin["replays"] < 500):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        g.replay()
        s1.record(stream)
        torch.cuda.synchronize()
        spin["replays"] += 1
        spin["gpu_ms"] += s0.elapsed_time(s1)
    time_steps_graph.spin_up = {"replays": spin["replays"], "gpu_ms": round(spin["gpu_ms"], 2)}

    def one():
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        flush.fill()
        if g_warm is not None:
            g_warm.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        w0 = time.perf_counter()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - w0

    runs = [one() for _ in range(max(1, repeats))]
    del flush
    return statistics.median(r[0] for r in runs), runs[0][1], [r[0] for r in runs]


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


def byte_split(wl):
    """(read, written) algorithmic bytes of one expand call: inputs, each
    distinct adapter's weights and (add_inputs) the prior output are read,
    the slice windows of active rows written."""
    from sgmv_workloads import DTYPE_BYTES
    total, t_act, distinct = byte_model(wl)
    ob = DTYPE_BYTES[wl.out_dtype]
    written = sum(t_act * s.N * ob for s in wl.slices)
    return total - written, written


def _stream_library():
    import ctypes
    path = os.path.join(ROOT, "segmented_gather_gemm_amd", "libsgmv_stream.so")
    lib = ctypes.CDLL(path)
    lib.sgmv_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.sgmv_stream_probe.restype = ctypes.c_int
    return lib


def stream_ceilings(read_bytes, write_bytes, reps=20,
                    shapes=((1024, 1), (2048, 1), (4096, 1), (8192, 1), (1024, 4), (2048, 4),
                            (4096, 4))):
    """Streaming ceilings for a traffic of `read_bytes` read and
    `write_bytes` written per launch, from the hand-written probe kernel in
    libsgmv_stream.so (16-byte buffer accesses, non-temporal loads,
    non-temporal device-scope stores -- the SGMV kernels' forms): GB/s of
    the reads alone, of the writes alone, and of both in one launch with the
    reads spread evenly among the writes.  Each figure is the best over a
    few launch shapes (grid size, accesses in flight per thread) of `reps`
    back-to-back launches, each on the next of
    enough buffer copies that no launch finds its data in the caches (1 GiB
    and more).  Context for the HBM roofline, not the metric."""
    import torch
    lib = _stream_library()
    R = (int(read_bytes) // 16) * 16
    Wb = (int(write_bytes) // 16) * 16
    limit = (1 << 31) - 16
    R, Wb = min(R, limit), min(Wb, limit)
    sets = max(2, math.ceil((1 << 30) / max(1, R + Wb)))
    src = [torch.ones(max(R, 16) // 4, dtype=torch.int32, device="cuda") for _ in range(sets)]
    dst = [torch.empty(max(Wb, 16) // 4, dtype=torch.int32, device="cuda") for _ in range(sets)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def rate(rb, wb):
        if rb + wb == 0:
            return None
        best = 0.0
        for blocks, unroll in shapes:
            def launch(i):
                rc = lib.sgmv_stream_probe(src[i % sets].data_ptr(), rb, dst[i % sets].data_ptr(),
                                           wb, sink.data_ptr(), blocks, unroll, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"stream probe failed with HIP error {rc}")
            for i in range(3):
                launch(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            best = max(best, (rb + wb) / (ms * 1e-3) / 1e9)
        return round(best, 1)

    out = {"read_bytes": R, "write_bytes": Wb, "read_gbs": rate(R, 0),
           "write_gbs": rate(0, Wb), "mix_gbs": rate(R, Wb)}
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


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


def shrink_byte_split(wl):
    """(read, written) algorithmic bytes of one shrink call."""
    from sgmv_workloads import DTYPE_BYTES
    total, t_act, _ = shrink_byte_model(wl)
    written = len(wl.lora_a) * t_act * wl.K * DTYPE_BYTES[wl.out_dtype]
    return total - written, written


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
    replays = None
    if args.eager:
        ms, wall, mode = ms_eager, wall_eager, "eager"
    else:
        log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (HIP-graph replay)")
        ms, wall, replays = time_steps_graph(step, args.steps, args.warmup)
        mode = "hip-graph replay (median of 5 timed replays of the K steps)"
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
    del sets, first
    torch.cuda.empty_cache()
    ceilings = None
    if not args.no_ceiling:
        log("bench: streaming ceilings for the same read / write traffic")
        rb, wb = shrink_byte_split(wl)
        ceilings = stream_ceilings(rb, wb)
        ceilings["pct_of_mix"] = round(100 * gbs / ceilings["mix_gbs"], 1)
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
            "workspace": "the binding's shared per-device buffer (balanced split-T batches)",
            "launch": mode,
            "timed_replays_us_per_step": None if replays is None else [round(r * 1e3, 3) for r in replays],
            "untimed_spin_up": None if replays is None else getattr(time_steps_graph, "spin_up", None),
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
        "streaming_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# Fused LoRA delta (shrink and expand in one launch) workloads.
# ---------------------------------------------------------------------------

def fused_byte_model(wl):
    """Algorithmic bytes of one fused call: the input rows of active
    segments, each distinct adapter's lora_A and lora_B rows once per slice,
    the windows of active rows written (and read, with add_inputs); the
    projection never leaves the chip.  Returns (total, read, T_act,
    distinct)."""
    from sgmv_workloads import DTYPE_BYTES
    act = wl.active_mask()
    t_act = int(wl.lens[act].sum())
    distinct = len(set(wl.idx[act].tolist()))
    wb, ob = DTYPE_BYTES[wl.w_dtype], DTYPE_BYTES[wl.out_dtype]
    n_total = sum(b.shape[1] for b in wl.lora_b)
    read = t_act * wl.H * DTYPE_BYTES[wl.x_dtype]
    read += distinct * len(wl.lora_a) * wl.K * wl.H * wb + distinct * n_total * wl.K * wb
    read += t_act * n_total * ob if wl.add else 0
    written = t_act * n_total * ob
    return read + written, read, t_act, distinct


class FusedBufferSet:
    def __init__(self, wl, device):
        import numpy as np
        import torch
        from sgmv_workloads import to_torch
        self.x = to_torch(wl.x, wl.x_dtype, device)
        self.a = [to_torch(np.ascontiguousarray(a).reshape(a.shape[0], -1), wl.w_dtype,
                           device).view(a.shape) for a in wl.lora_a]
        self.b = [to_torch(np.ascontiguousarray(b).reshape(b.shape[0], -1), wl.w_dtype,
                           device).view(b.shape) for b in wl.lora_b]
        self.out = to_torch(wl.out0, wl.out_dtype, device)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[wl.w_dtype]
        self.y = [torch.zeros((wl.T, wl.K), dtype=tdt, device=device) for _ in wl.lora_a]

    def clone(self):
        c = object.__new__(FusedBufferSet)
        c.x = self.x.clone()
        c.a = [t.clone() for t in self.a]
        c.b = [t.clone() for t in self.b]
        c.out = self.out.clone()
        c.y = [t.clone() for t in self.y]
        return c


def make_fused_step(wl, meta, sets, unfused=False):
    """One step: one sgmv_fused_shrink_expand call, or with `unfused` the
    two-launch pair it replaces (sgmv_shrink_multi_slice into weight-dtype
    projections, then sgmv_expand_multi_slice of them)."""
    import segmented_gather_gemm_amd as sg
    start, lens, idx = meta
    B, M = wl.batches, wl.max_seq_len
    if unfused:
        def step(i):
            bs = sets[i % len(sets)]
            sg.sgmv_shrink_multi_slice(bs.x, list(zip(bs.a, bs.y)), start, lens, idx, B, M,
                                       wl.scale)
            sg.sgmv_expand_multi_slice(list(zip(bs.y, bs.b, wl.offsets)), bs.out, start, lens,
                                       idx, B, M, wl.add)
    else:
        def step(i):
            bs = sets[i % len(sets)]
            sg.sgmv_fused_shrink_expand(bs.x, list(zip(bs.a, bs.b, wl.offsets)), bs.out, start,
                                        lens, idx, B, M, wl.scale, wl.add)
    return step


def fused_cpu_baseline(wl, budget_s):
    """Time the oracle's fused reference (shrink, then expand; as it stands)
    on a bounded sample: the first segments, as many as about `budget_s`
    seconds of work on all host cores allow; then a smaller sample on one
    core."""
    import numpy as np
    import oracle
    import sgmv_workloads as W
    threads = len(os.sched_getaffinity(0))
    n_total = sum(b.shape[1] for b in wl.lora_b)
    macs_row = len(wl.lora_a) * wl.K * wl.H + n_total * wl.K

    def sample_for(seconds, nthreads):
        # estimate: ~1e8 fp64 multiply-adds per second per thread
        act = wl.active_mask()
        macs = int(wl.lens[act].sum()) * macs_row
        if macs / (1e8 * nthreads) <= seconds:
            return wl, "full workload"
        keep = max(1, int(len(wl.lens) * seconds * 1e8 * nthreads / macs))
        idx = wl.idx.copy()
        idx[keep:] = -1
        smp = W.FusedWorkload(wl.name, wl.x, wl.x_dtype, wl.lora_a, wl.lora_b, wl.w_dtype,
                              wl.offsets, wl.out0, wl.out_dtype, wl.start, wl.lens, idx,
                              wl.scale, wl.add, wl.K, wl.L, wl.seed)
        return smp, f"first {keep} of {len(wl.lens)} segments"

    def run(sample, nthreads, seconds, max_reps):
        reps, spent = 0, 0.0
        while reps == 0 or (spent < seconds and reps < max_reps):
            out = sample.out0.copy()
            t0 = time.perf_counter()
            oracle.fused(sample.x, sample.x_dtype, sample.lora_a, sample.lora_b, sample.w_dtype,
                         sample.offsets, out, sample.out_dtype, sample.start, sample.lens,
                         sample.idx, sample.scale, sample.add, threads=nthreads)
            spent += time.perf_counter() - t0
            reps += 1
        return spent / reps, reps

    sample, note = sample_for(budget_s, threads)
    secs, reps = run(sample, threads, budget_s, 1000)
    sample_bytes = fused_byte_model(sample)[0]
    one, one_note = sample_for(budget_s / 4, 1)
    secs1, _ = run(one, 1, 0.0, 1)
    one_bytes = fused_byte_model(one)[0]
    return {"value": round(sample_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_call": round(secs, 4), "reps": reps,
            "sample": f"{note} of {wl.name} seed {wl.seed}, fp64 C oracle, {reps} calls",
            "single_core_gbs": round(one_bytes / secs1 / 1e9, 4),
            "single_core_sample": f"{one_note}, one call"}


def run_fused(args):
    import torch
    import sgmv_workloads as W
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    log(f"bench: generating {args.workload} seed {args.seed}")
    wl = W.FUSED_WORKLOADS[args.workload](args.seed)
    model_bytes, read_bytes, t_act, distinct = fused_byte_model(wl)
    fp = (wl.x.nbytes + sum(a.nbytes for a in wl.lora_a) + sum(b.nbytes for b in wl.lora_b) +
          wl.out0.nbytes)
    nsets = rotated_sets(fp)
    log(f"bench: {len(wl.lora_a)} slice(s), T={wl.T} (active {t_act}), hidden {wl.H} -> rank "
        f"{wl.K} -> {[b.shape[1] for b in wl.lora_b]}, {distinct} distinct adapters, "
        f"{model_bytes / 1e6:.2f} MB per call, {nsets} rotated buffer sets of {fp / 1e6:.1f} MB")
    meta = tuple(torch.from_numpy(a).to(device) for a in (wl.start, wl.lens, wl.idx))
    first = FusedBufferSet(wl, device)
    sets = [first] + [first.clone() for _ in range(nsets - 1)]
    torch.cuda.synchronize()
    step = make_fused_step(wl, meta, sets, args.unfused)

    log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (eager launches)")
    ms_eager, wall_eager = time_steps(step, args.steps, args.warmup)
    log(f"bench: eager {ms_eager * 1e3:.2f} us per step")
    replays = None
    if args.eager:
        ms, wall, mode = ms_eager, wall_eager, "eager"
    else:
        log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (HIP-graph replay)")
        ms, wall, replays = time_steps_graph(step, args.steps, args.warmup)
        mode = "hip-graph replay (median of 5 timed replays of the K steps)"
    log("bench: single launches after a cache flush")
    ms_single = time_single_launches(step)
    sec = ms * 1e-3
    gbs = model_bytes / sec / 1e9
    tokens_s = wl.T / sec
    ksha = kernel_source_hash("fused")
    traffic_bytes = None if args.unfused else traffic_from_profiles(args.workload, ksha)
    traffic = None if traffic_bytes is None else round(traffic_bytes / sec / 1e9, 2)
    log(f"bench: {ms * 1e3:.2f} us per step, {gbs:.1f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% "
        f"of peak), {tokens_s / 1e6:.2f} M tokens/s (wall {wall:.2f} s)")
    del sets, first
    torch.cuda.empty_cache()
    ceilings = None
    if not args.no_ceiling:
        log("bench: streaming ceilings for the same read / write traffic")
        ceilings = stream_ceilings(read_bytes, model_bytes - read_bytes)
        ceilings["pct_of_mix"] = round(100 * gbs / ceilings["mix_gbs"], 1)
    cpu = None
    if args.cpu_budget > 0:
        log("bench: timing the CPU oracle baseline")
        cpu = fused_cpu_baseline(wl, args.cpu_budget)
    result = {
        "metric": "effective HBM GB/s (% of MI355X peak) and tokens/s for sgmv_fused_shrink_expand",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.w_dtype,
        "data": "synthetic",
        "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(tokens_s, 1),
        "config": {
            "workload": args.workload,
            "seed": args.seed,
            "hidden": wl.H,
            "rank": wl.K,
            "slices": [[o, b.shape[1]] for o, b in zip(wl.offsets, wl.lora_b)],
            "batches": wl.batches,
            "total_tokens": wl.T,
            "active_tokens": t_act,
            "distinct_adapters": distinct,
            "scale": wl.scale,
            "add_inputs": wl.add,
            "dtypes": {"inputs": wl.x_dtype, "lora_a_b": wl.w_dtype, "output": wl.out_dtype,
                       "projection": wl.w_dtype, "accumulate": "f32"},
            "bytes_per_step": model_bytes,
            "rotated_buffer_sets": nsets,
            "call": ("sgmv_shrink_multi_slice + sgmv_expand_multi_slice" if args.unfused else
                     "sgmv_fused_shrink_expand"),
            "workspace": ("the shrink's: the binding's shared per-device buffer" if args.unfused
                          else None),
            "launch": mode,
            "timed_replays_us_per_step": None if replays is None else [round(r * 1e3, 3) for r in replays],
            "untimed_spin_up": None if replays is None else getattr(time_steps_graph, "spin_up", None),
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
            "kernel": "two launches" if args.unfused else "fused_shrink_expand",
            "kernel_source_sha256_16": ksha,
        },
        "streaming_ceilings": ceilings,
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
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-ceiling probes")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (default: HIP-graph replay, eager also reported)")
    ap.add_argument("--unfused", action="store_true",
                    help="fused workloads: time the two-launch pair (shrink, then expand) "
                         "instead of the fused call")
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
    if args.workload in W.FUSED_WORKLOADS:
        return run_fused(args)
    if args.workload not in W.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from "
                 f"{sorted(W.WORKLOADS) + sorted(W.SHRINK_WORKLOADS) + sorted(W.FUSED_WORKLOADS)}")
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    log(f"bench: generating {args.workload} seed {args.seed}")
    wl = W.WORKLOADS[args.workload](args.seed)
    model_bytes, t_act, distinct = byte_model(wl)
    fp = footprint_bytes(wl)
    nsets = rotated_sets(fp)
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
    replays = None
    if args.eager:
        ms, wall, mode = ms_eager, wall_eager, "eager"
    else:
        log(f"bench: {args.warmup} warm-up + {args.steps} timed steps (HIP-graph replay)")
        ms, wall, replays = time_steps_graph(step, args.steps, args.warmup)
        mode = "hip-graph replay (median of 5 timed replays of the K steps)"
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

    del sets, first
    torch.cuda.empty_cache()
    ceilings = None
    if not args.no_ceiling:
        log("bench: streaming ceilings for the same read / write traffic")
        rb, wb = byte_split(wl)
        ceilings = stream_ceilings(rb, wb)
        ceilings["pct_of_mix"] = round(100 * gbs / ceilings["mix_gbs"], 1)

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
            "timed_replays_us_per_step": None if replays is None else [round(r * 1e3, 3) for r in replays],
            "untimed_spin_up": None if replays is None else getattr(time_steps_graph, "spin_up", None),
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
        "streaming_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
