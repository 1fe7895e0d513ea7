#!/usr/bin/env python3
"""Benchmark of the MoE dispatch-preprocessing hot path on one MI355X.

One step is one pass of the receive-side path over one prefill batch:
moe_layout -> moe_scatter_quant -> moe_combine on T=8192 tokens,
hidden 7168, 256 local experts, top-8 routing from a Zipf(1.1) expert
popularity (8 experts never chosen), compact layout with 128-row blocks
(98048-row static bound), fp8 e4m3 with UE8M0 group-128 scales.  Inputs are
synthetic and already resident in HBM when the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  ``value`` is the step's algorithmic HBM bytes (what
the method must move: each token row read once, each local assignment's fp8
row and scales written once, each combined row read once, index and weight
tables, no padding rows) divided by the step time measured by wall clock
over the timed steps.  Kernel times come from HIP events recorded on the
stream the kernels run on, created with the system fence disabled so that
recording them does not flush the caches: one pair per step around the
combine inside the timed loop, and every kernel in a second pass.
``cpu_baseline`` times the CPU oracle on the same workload on this host.
The other rows of the path (masked decode slab, send-side live-row MX
quant, per-token -> per-tensor requant, large combine) are timed separately
under ``rows``; they are not part of ``value``.
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("dispatch scatter+quant+combine HBM GB/s (% of MI355X peak); "
          "assignments/sec")
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_prefill_traffic.txt")
COMBINE_SRC = os.path.join(ROOT, "fp8_mx_activation_amd", "csrc",
                           "combine.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu", action="store_true",
                   help="skip the CPU oracle baseline")
    p.add_argument("--no-rows", action="store_true",
                   help="skip the separately timed rows")
    p.add_argument("--cpu-repeats", type=int, default=3)
    p.add_argument("--samples", type=int, default=100,
                   help="samples behind each median and spread: steps of "
                        "the per-kernel and MALL-flushed passes, graph "
                        "replays and flushed calls of every row (fewer for "
                        "runs under a profiler)")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the step, time masked against compact "
                        "layouts over a range of token counts")
    return p.parse_args()


# ------------------------------------------------------------ byte counts

def bytes_layout(T, K, E, rows):
    # ids read, src2dst written, m_indices written, counts + masked_m +
    # region starts written
    return T * K * 4 + T * K * 4 + rows * 4 + E * 8 + (E + 1) * 4


def bytes_scatter(tokens_touched, T, K, H, G, assignments):
    return tokens_touched * H * 2 + assignments * (H + H // G) + T * K * 4


def bytes_combine(T, K, H, assignments, out_bytes=2):
    return assignments * H * 2 + T * K * 8 + T * H * out_bytes


# ---------------------------------------------------------------- helpers

def spread(samples):
    """Median, 10th and 90th percentile of a list of times (or rates)."""
    a = np.asarray(samples, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2),
            "median": round(float(np.median(a)), 2),
            "p90": round(float(np.percentile(a, 90)), 2),
            "n": int(a.size)}


def time_calls_samples(torch, fn, reps=20, warmup=3, replays=100):
    """GPU time per call of fn, in microseconds, one sample per replay: reps
    calls captured in one hipGraph, timed with events around each replay,
    so host launch cost between calls is not counted."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    hs = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2 * replays)
    for i in range(replays):
        ev.record(2 * i, hs)
        g.replay()
        ev.record(2 * i + 1, hs)
    torch.cuda.synchronize()
    per = [ev.ms(2 * i, 2 * i + 1) / reps * 1e3 for i in range(replays)]
    ev.close()
    del g
    return per


def time_calls(torch, fn, reps=20, warmup=3, replays=None):
    """Median of time_calls_samples."""
    replays = SAMPLES if replays is None else replays
    return float(np.median(time_calls_samples(torch, fn, reps, warmup,
                                              replays)))


def time_calls_cold_wb(torch, fn, flush, reps=100, warmup=2):
    """GPU time per call of fn with the 256 MB last-level cache (MALL) and
    the L2s flushed before each call by reading `flush` (512 MB, written
    once beforehand, so the evicting lines are clean and nothing is written
    back during the call); events bracket the call alone.  Lines the call
    leaves dirty in the MALL reach HBM only later, so a flush right after
    the call is timed against a flush after a flush, and the median of that
    difference (the write-back, at least 0) is added to every sample.
    Returns (samples in microseconds, write-back in microseconds)."""
    for _ in range(warmup):
        fn()
    flush_f = flush.view(torch.float32)
    torch.cuda.synchronize()
    hs = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(4 * reps)
    for i in range(reps):
        flush_f.sum()
        ev.record(4 * i, hs)
        fn()
        ev.record(4 * i + 1, hs)
        flush_f.sum()
        ev.record(4 * i + 2, hs)
        flush_f.sum()
        ev.record(4 * i + 3, hs)
    torch.cuda.synchronize()
    per = [ev.ms(4 * i, 4 * i + 1) * 1e3 for i in range(reps)]
    wb = max(0.0, float(np.median(
        [(ev.ms(4 * i + 1, 4 * i + 2) - ev.ms(4 * i + 2, 4 * i + 3)) * 1e3
         for i in range(reps)])))
    ev.close()
    return [p + wb for p in per], wb


def time_calls_cold_samples(torch, fn, flush, reps=100, warmup=2):
    """The samples of time_calls_cold_wb (write-back included)."""
    return time_calls_cold_wb(torch, fn, flush, reps, warmup)[0]


def time_calls_cold(torch, fn, flush, reps=100, warmup=2):
    """Median of time_calls_cold_samples."""
    return float(np.median(time_calls_cold_samples(torch, fn, flush, reps,
                                                   warmup)))


SAMPLES = 100  # set from --samples in main()

# output buffers a combine timing rotates over (see the step's setup)
N_OUT = 4
# token-row copies of the step with its rows read from HBM
N_X = 3


def rotation(bufs):
    """A function returning bufs[0], bufs[1], ... in turn, cyclically."""
    it = itertools.cycle(bufs)
    return lambda: next(it)


def timed_row(torch, fn, nbytes=None, units=None, unit_name=None, reps=20,
              replays=None, flush=None):
    """A row's record: median time per call with its 10-90 % spread over
    `replays` graph replays (and over as many calls with the MALL flushed
    when `flush` is given), plus GB/s of `nbytes` and `unit_name`/s."""
    replays = SAMPLES if replays is None else replays
    per = time_calls_samples(torch, fn, reps=reps, replays=replays)
    us = float(np.median(per))
    r = {"us": round(us, 2), "us_spread": spread(per)}
    if nbytes is not None:
        r["algorithmic_bytes"] = nbytes
        r["gbs"] = round(nbytes / (us * 1e-6) / 1e9, 2)
    if units is not None:
        r[unit_name + "_per_s"] = round(units / (us * 1e-6), 1)
    if flush is not None:
        cold, wb = time_calls_cold_wb(torch, fn, flush, reps=replays)
        cu = float(np.median(cold))
        r["cold_us"] = round(cu, 2)
        r["cold_us_spread"] = spread(cold)
        r["cold_write_back_us"] = round(wb, 2)
        if nbytes is not None:
            r["cold_gbs"] = round(nbytes / (cu * 1e-6) / 1e9, 2)
    return r


class HipEvents:
    """Timing events on a given HIP stream, created through the HIP runtime
    the process has loaded, with hipEventDisableSystemFence.

    A default event (torch.cuda.Event included) does a system-scope release
    when it completes: the L2s are written back and invalidated, which costs
    a few microseconds per record and slows the next kernel.  On this
    workload four such events per step add about 14 us to a 280 us step;
    with the fence disabled four events add about 7 us and two about half
    of that.  The events are only read for elapsed times after a device
    synchronization, which is all the flag requires."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self._ct = ctypes
        self._hip = ctypes.CDLL(path or "libamdhip64.so")
        h = self._hip
        h.hipEventCreateWithFlags.argtypes = [
            ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [
            ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = h.hipEventCreateWithFlags(ctypes.byref(e),
                                           self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
            self.ev.append(e)
        self.record_fn = h.hipEventRecord

    def record(self, i, stream):
        return self.record_fn(self.ev[i], stream)

    def ms(self, i, j):
        f = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(f), self.ev[i],
                                           self.ev[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return f.value

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def graph_step_ms(torch, fn, warmup, steps, per_graph=1):
    """Capture fn(0), ..., fn(per_graph - 1) once in a hipGraph; time
    replays covering `steps` steps; milliseconds per step."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(per_graph):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    n = max(1, steps // per_graph)
    for _ in range(max(1, warmup // per_graph)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / (n * per_graph)


def traffic_record():
    """HBM bytes per combine launch from committed rocprofv3 counters, or
    None if absent or taken on another version of the kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    src = hashlib.sha256(open(COMBINE_SRC, "rb").read()).hexdigest()
    if kv.get("combine_source_sha256") != src:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------- main

def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write(
            "bench.py runs on one GPU only: the path is measured on one GPU's "
            "share of the experts at its real shape (--gpus 1); multi-GPU "
            "runs are not part of this benchmark.\n")
        sys.exit(2)

    import torch

    import fp8_mx_activation_amd as mxq
    import synthetic_inputs as si

    global SAMPLES
    SAMPLES = max(1, args.samples)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.sweep:
        print(json.dumps(layout_sweep(torch, mxq, si, dev)), flush=True)
        return

    # ---------------------------------------------------------- inputs
    b = si.prefill_compact()
    T, H, K, E, G = b.T, b.H, b.K, b.n_local, b.group
    R = mxq.moe_compact_row_bound(T * K, E, b.block_e)
    x = torch.from_numpy(b.x.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.from_numpy(b.topk_ids).to(dev)
    w = torch.from_numpy(b.topk_weights).to(dev)
    y = si.gaussian_bf16_device(303, (R, H), dev)   # expert outputs
    lay_out = {k: torch.empty(s, dtype=torch.int32, device=dev)
               for k, s in (("counts", (E,)), ("expert_offsets", (E + 1,)),
                            ("m_indices", (R,)), ("masked_m", (E,)),
                            ("src2dst", (T, K)), ("overflow_flag", (1,)))}
    ws = torch.empty(max(1, mxq.moe_layout_workspace_bytes(T, K, E)),
                     dtype=torch.uint8, device=dev)
    q = torch.empty((R, H), dtype=torch.uint8, device=dev)
    s = torch.empty((R, H // G), dtype=torch.uint8, device=dev)
    # The combine's output rotates over N_OUT buffers (470 MB, more than the
    # 256 MB MALL) in every warm timing: its device-scope stores leave lines
    # dirty in the MALL, and one buffer rewritten every step could be
    # overwritten there without ever reaching HBM.  With four, a buffer's
    # lines are written back before the step that writes it again.
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            for _ in range(N_OUT)]
    out = outs[0]

    local = ((b.topk_ids >= 0) & (b.topk_ids < E))
    A = int(local.sum())
    touched = int(local.any(axis=1).sum())
    B_lay = bytes_layout(T, K, E, R)
    B_sq = bytes_scatter(touched, T, K, H, G, A)
    B_cb = bytes_combine(T, K, H, A)
    B_step = B_lay + B_sq + B_cb

    # box copy bandwidth (device-to-device copy, read + write bytes)
    cbuf_a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cbuf_b = torch.empty_like(cbuf_a)
    copy_us = time_calls(torch, lambda: cbuf_b.copy_(cbuf_a), reps=10)
    copy_gbs = 2 * cbuf_a.numel() / (copy_us * 1e-6) / 1e9
    # the same copy with the library's 16-byte vector copy kernel
    copy16 = {}
    for mode, name in ((0, "plain"), (1, "nontemporal_stores"),
                       (3, "nontemporal_loads_and_stores")):
        us = time_calls(torch, lambda: mxq.mxq_copy16(cbuf_a, cbuf_b, mode),
                        reps=10)
        copy16[name] = round(2 * cbuf_a.numel() / (us * 1e-6) / 1e9, 1)
    del cbuf_a, cbuf_b

    def step(i=0):
        lay = mxq.moe_layout(ids, 0, E, "compact", num_rows=R, out=lay_out,
                             workspace=ws)
        mxq.moe_scatter_quant(x, lay["src2dst"], R, "ue8m0_g128", q=q,
                              scales=s)
        mxq.moe_combine(y, lay["src2dst"], w, out=outs[i % N_OUT])

    # The timed loop calls the C entry points directly with arguments
    # prepared once (the same calls the wrappers above make), and its events
    # are created beforehand, so the host issues a step in a few
    # microseconds and stays ahead of the GPU.
    L = mxq.lib()
    hs = torch.cuda.current_stream().cuda_stream
    p = {k: t.data_ptr() for k, t in lay_out.items()}
    lay_args = (ids.data_ptr(), T, K, 0, E, mxq.LAYOUT_KINDS["compact"],
                b.block_e, 0, R, p["counts"], p["expert_offsets"],
                p["m_indices"], p["masked_m"], p["src2dst"],
                p["overflow_flag"], ws.data_ptr(), ws.numel(), hs)
    sq_args = (x.data_ptr(), H, T, H, p["src2dst"], K,
               mxq.SCALE_FORMATS["ue8m0_g128"][0], q.data_ptr(), H,
               s.data_ptr(), H // G, R, hs)
    cb_argv = [(y.data_ptr(), H, R, p["src2dst"], w.data_ptr(), T, K, H,
                o.data_ptr(), H, mxq.OUT_DTYPES[torch.bfloat16], hs)
               for o in outs]
    # Timing events are HIP events on the launch stream with the system
    # fence disabled (HipEvents).  The timed region holds one pair per step,
    # around the combine (the roofline kernel); the layout and scatter times
    # come from a second pass of the same steps with a pair around every
    # kernel, since each event adds a little time to the step it sits in.
    hev = HipEvents(2 * args.steps)

    def step_fast(i):
        st = L.moe_layout(*lay_args)
        st |= L.moe_scatter_quant(*sq_args)
        st |= hev.record(2 * i, hs)
        st |= L.moe_combine(*cb_argv[i % N_OUT])
        st |= hev.record(2 * i + 1, hs)
        return st

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    status = 0
    t0 = time.perf_counter()
    for i in range(args.steps):
        status |= step_fast(i)
    t_issue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    if status != 0:
        raise RuntimeError("a library call in the timed loop failed "
                           "(status bits %d)" % status)
    cb_ms = [hev.ms(2 * i, 2 * i + 1) for i in range(args.steps)]
    hev.close()
    step_ms = wall_s * 1e3 / args.steps

    # the same steps with no event at all, to show what the roofline's
    # events cost the timed loop (reported beside value, not as value)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        status |= L.moe_layout(*lay_args)
        status |= L.moe_scatter_quant(*sq_args)
        status |= L.moe_combine(*cb_argv[i % N_OUT])
    torch.cuda.synchronize()
    noev_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if status != 0:
        raise RuntimeError("a library call in the event-free pass failed")

    # the same steps with the token rows rotating over N_X copies (351 MB,
    # more than the MALL), so that every step's scatter reads its rows from
    # HBM: wall clock, no events, no flushes -- the steady state when the
    # activations handed over are no longer cached
    xs = [x] + [x.clone() for _ in range(N_X - 1)]
    sq_argv = [(xx.data_ptr(),) + sq_args[1:] for xx in xs]
    for i in range(2 * N_X * N_OUT):
        status |= L.moe_layout(*lay_args)
        status |= L.moe_scatter_quant(*sq_argv[i % N_X])
        status |= L.moe_combine(*cb_argv[i % N_OUT])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        status |= L.moe_layout(*lay_args)
        status |= L.moe_scatter_quant(*sq_argv[i % N_X])
        status |= L.moe_combine(*cb_argv[i % N_OUT])
    torch.cuda.synchronize()
    hbm_rows_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if status != 0:
        raise RuntimeError("a library call in the rotating-rows pass failed")
    del xs, sq_argv

    # per-kernel pass: the same steps with events around each kernel, at
    # least 100 of them whatever --steps is, for the spread of each kernel
    n_k = max(args.steps, args.samples)
    kev = HipEvents(4 * n_k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_k):
        status |= kev.record(4 * i, hs)
        status |= L.moe_layout(*lay_args)
        status |= kev.record(4 * i + 1, hs)
        status |= L.moe_scatter_quant(*sq_args)
        status |= kev.record(4 * i + 2, hs)
        status |= L.moe_combine(*cb_argv[i % N_OUT])
        status |= kev.record(4 * i + 3, hs)
    torch.cuda.synchronize()
    kev_step_ms = (time.perf_counter() - t0) * 1e3 / n_k
    if status != 0:
        raise RuntimeError("a library call in the per-kernel pass failed")
    k_us = [[kev.ms(4 * i + k, 4 * i + k + 1) * 1e3 for i in range(n_k)]
            for k in range(3)]
    kev.close()
    lay_us, sq_us, kcb_us = k_us
    ev_step_ms = float(np.mean(lay_us) + np.mean(sq_us) +
                       np.mean(kcb_us)) / 1e3

    # the same step captured once in a hipGraph and replayed (no per-kernel
    # host launch cost); reported beside the eager timed region
    graph_ms = graph_step_ms(torch, step, args.warmup, args.steps, N_OUT)

    # The same step with the 256 MB last-level cache (MALL) and the L2s
    # flushed before each step by reading 512 MB, so that every input comes
    # from HBM (in the loop above the token rows stay cached from the
    # previous step, since the combine's loads bypass the cache); events
    # bracket the step's kernels.  Lines the step leaves dirty in the MALL
    # (the combine's device-scope stores end there) reach HBM only later;
    # that write-back is charged to the step: a second flush right after the
    # step is timed against a third one, which finds nothing to write back.
    flush = torch.zeros(512 << 20, dtype=torch.uint8,
                        device=dev).view(torch.float32)
    n_cold = args.samples
    evc = HipEvents(6 * n_cold)
    torch.cuda.synchronize()
    for i in range(n_cold):
        flush.sum()
        status |= evc.record(6 * i, hs)
        status |= L.moe_layout(*lay_args)
        status |= evc.record(6 * i + 1, hs)
        status |= L.moe_scatter_quant(*sq_args)
        status |= evc.record(6 * i + 2, hs)
        status |= L.moe_combine(*cb_argv[i % N_OUT])
        status |= evc.record(6 * i + 3, hs)
        flush.sum()
        status |= evc.record(6 * i + 4, hs)
        flush.sum()
        status |= evc.record(6 * i + 5, hs)
    torch.cuda.synchronize()
    if status != 0:
        raise RuntimeError("a library call in the flushed loop failed")
    cold_us = [[evc.ms(6 * i + k, 6 * i + k + 1) * 1e3 for i in range(n_cold)]
               for k in range(3)]
    # per step: the flush after it minus a flush after a flush
    wb_us = [(evc.ms(6 * i + 3, 6 * i + 4) - evc.ms(6 * i + 4, 6 * i + 5)) *
             1e3 for i in range(n_cold)]
    evc.close()

    # The combine's two halves alone, in this run: its gather reads (the
    # same 65536 rows through the same src2dst, non-temporal loads) and its
    # 117 MB of output rows written with streaming stores; their sum is the
    # time the combine would take if its reads and writes simply added up.
    # Successive calls write the rotating output buffers in turn.
    gather_sink = torch.empty(T, dtype=torch.int32, device=dev)
    s2d = lay_out["src2dst"]
    ns = args.samples
    gather_us = time_calls_samples(
        torch, lambda: mxq.mxq_gather_read16(y, s2d, gather_sink),
        replays=ns)
    nxt = rotation(outs)
    write_us = time_calls_samples(
        torch, lambda: mxq.mxq_fill_rows16(nxt()), replays=ns)
    comb_us_graph = time_calls_samples(
        torch, lambda: mxq.moe_combine(y, s2d, w, out=nxt()), replays=ns)
    # the same three with the MALL flushed before each call
    gather_cold = time_calls_cold_samples(
        torch, lambda: mxq.mxq_gather_read16(y, s2d, gather_sink), flush,
        reps=ns)
    write_cold = time_calls_cold_samples(
        torch, lambda: mxq.mxq_fill_rows16(nxt()), flush, reps=ns)
    del flush

    value = B_step / (step_ms * 1e-3) / 1e9
    cb_gbs = B_cb / (np.mean(cb_ms) * 1e-3) / 1e9
    sq_gbs = B_sq / (np.median(sq_us) * 1e-6) / 1e9
    kcb_gbs = B_cb / (np.median(kcb_us) * 1e-6) / 1e9
    sqcb_gbs = ((B_sq + B_cb) / ((np.median(sq_us) + np.median(kcb_us)) *
                                 1e-6) / 1e9)
    # per flushed step: scatter+combine as a fraction of the 8 TB/s peak,
    # with the write-back the step left charged to it
    wb_med = max(0.0, float(np.median(wb_us)))
    frac_cold = [(B_sq + B_cb) / ((a + c + wb_med) * 1e-6) / 1e9 /
                 PEAK_HBM_GBS for a, c in zip(cold_us[1], cold_us[2])]
    frac_cold_nowb = [(B_sq + B_cb) / ((a + c) * 1e-6) / 1e9 / PEAK_HBM_GBS
                      for a, c in zip(cold_us[1], cold_us[2])]
    frac_warm = [(B_sq + B_cb) / ((a + c) * 1e-6) / 1e9 / PEAK_HBM_GBS
                 for a, c in zip(sq_us, kcb_us)]
    cold_med = [float(np.median(c)) for c in cold_us]
    cold_step_us = sum(cold_med) + wb_med
    traffic = traffic_record()
    g_med, w_med = float(np.median(gather_us)), float(np.median(write_us))
    c_med = float(np.median(comb_us_graph))

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "prefill compact dispatch: T=8192 tokens, hidden "
                        "7168, 256 local experts, top-8 Zipf(1.1) routing "
                        "(8 experts empty), compact layout block 128 "
                        "(98048-row bound), fp8 e4m3 + UE8M0 group-128; "
                        "step = moe_layout + moe_scatter_quant + moe_combine",
            "tokens": T, "hidden": H, "local_experts": E, "topk": K,
            "assignments": A, "layout_rows": R, "group": G,
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "assignments_per_s": round(A / (step_ms * 1e-3), 1),
        "host_issue_ms_per_step": round(t_issue * 1e3 / args.steps, 4),
        "graph_replay": {"ms_per_step": round(graph_ms, 4),
                         "gbs": round(B_step / (graph_ms * 1e-3) / 1e9, 2)},
        "timing": "value: wall clock over the timed steps, bracketed by "
                  "device synchronizations, with the token rows still in "
                  "the MALL from the previous step; HIP events (system "
                  "fence disabled) on the launch stream around each step's "
                  "combine in the same loop give the roofline; the "
                  "per-kernel pass (>= 100 steps) and the MALL-flushed pass "
                  "(100 steps) bracket every kernel; spreads are the 10th, "
                  "50th and 90th percentiles over those samples",
        "moe_combine_us_in_timed_region": round(
            1e3 * float(np.mean(cb_ms)), 2),
        "ms_per_step_without_events": round(noev_step_ms, 4),
        "step_token_rows_from_hbm": {
            "note": "the same steps by wall clock, without events, with the "
                    "token rows rotating over %d copies (more than the 256 "
                    "MB MALL) so that every scatter reads them from HBM" %
                    N_X,
            "ms_per_step": round(hbm_rows_step_ms, 4),
            "gbs": round(B_step / (hbm_rows_step_ms * 1e-3) / 1e9, 2),
            "pct_of_peak": round(
                100 * B_step / (hbm_rows_step_ms * 1e-3) / 1e9 /
                PEAK_HBM_GBS, 2),
        },
        "scatter_quant_plus_combine": {
            "bytes": B_sq + B_cb,
            "us": round(float(np.median(sq_us) + np.median(kcb_us)), 2),
            "gbs": round(sqcb_gbs, 2),
            "pct_of_peak": round(100 * sqcb_gbs / PEAK_HBM_GBS, 2),
            "pct_of_peak_spread": spread([100 * f for f in frac_warm]),
        },
        "kernels_us": {
            "moe_layout": round(float(np.median(lay_us)), 2),
            "moe_scatter_quant": round(float(np.median(sq_us)), 2),
            "moe_combine": round(float(np.median(kcb_us)), 2),
            "event_sum_per_step": round(1e3 * ev_step_ms, 2),
            "ms_per_step_with_these_events": round(kev_step_ms, 4),
        },
        "kernels_us_spread": {"moe_layout": spread(lay_us),
                              "moe_scatter_quant": spread(sq_us),
                              "moe_combine": spread(kcb_us)},
        "kernels_gbs": {"moe_scatter_quant": round(sq_gbs, 2),
                        "moe_combine": round(kcb_gbs, 2)},
        "algorithmic_bytes": {"moe_layout": B_lay, "moe_scatter_quant": B_sq,
                              "moe_combine": B_cb, "step": B_step},
        "step_mall_flushed": {
            "note": "the MALL and L2s flushed (512 MB read) before each "
                    "step; HIP events around the step's kernels; the "
                    "write-back the step leaves in the MALL charged to it "
                    "(a flush after the step timed against a flush after "
                    "a flush); %d steps, medians" % n_cold,
            "ms_per_step": round(cold_step_us / 1e3, 4),
            "gbs": round(B_step / (cold_step_us * 1e-6) / 1e9, 2),
            "pct_of_peak": round(
                100 * B_step / (cold_step_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                2),
            "write_back_after_step_us": round(wb_med, 2),
            "ms_per_step_without_write_back": round(sum(cold_med) / 1e3, 4),
            "kernels_us": {"moe_layout": round(cold_med[0], 2),
                           "moe_scatter_quant": round(cold_med[1], 2),
                           "moe_combine": round(cold_med[2], 2)},
            "kernels_us_spread": {"moe_layout": spread(cold_us[0]),
                                  "moe_scatter_quant": spread(cold_us[1]),
                                  "moe_combine": spread(cold_us[2])},
            "scatter_quant_plus_combine_pct_of_peak": round(
                100 * float(np.median(frac_cold)), 2),
            "scatter_quant_plus_combine_pct_of_peak_spread": spread(
                [100 * f for f in frac_cold]),
            "scatter_quant_plus_combine_pct_of_peak_without_write_back":
                round(100 * float(np.median(frac_cold_nowb)), 2),
        },
        "box_copy_gbs": round(copy_gbs, 1),
        "box_copy16_kernel_gbs": copy16,
        "roofline": {
            "bound": "hbm",
            "kernel": "moe_combine",
            "achieved": round(cb_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(cb_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            # the target as the pages' workload defines it: scatter+quant
            # plus combine at the prefill shape, against the 8 TB/s peak
            "target_scatter_quant_plus_combine": {
                "frac_warm": round(float(np.median(frac_warm)), 4),
                "frac_mall_flushed": round(float(np.median(frac_cold)), 4),
                "frac_mall_flushed_p10": round(
                    float(np.percentile(frac_cold, 10)), 4),
                "frac_mall_flushed_p90": round(
                    float(np.percentile(frac_cold, 90)), 4),
            },
            # the best copy kernel of this run (16-byte vectors,
            # non-temporal loads and stores, 1 GiB read + 1 GiB written):
            # the rate the box sustains on a 1:1 read/write mix
            "same_run_copy_bound": {
                "copy16_gbs": copy16["nontemporal_loads_and_stores"],
                "combine_gbs": round(cb_gbs, 2),
                "combine_over_copy": round(
                    cb_gbs / copy16["nontemporal_loads_and_stores"], 4),
            },
            # the combine beside its own two halves measured in this run
            "combine_same_run_halves": {
                "gather_read_us": round(g_med, 2),
                "gather_read_gbs": round(
                    (A * H * 2 + T * K * 4) / (g_med * 1e-6) / 1e9, 2),
                "output_write_us": round(w_med, 2),
                "output_write_gbs": round(T * H * 2 / (w_med * 1e-6) / 1e9,
                                          2),
                "sum_us": round(g_med + w_med, 2),
                "combine_us": round(c_med, 2),
                "combine_over_sum": round(c_med / (g_med + w_med), 4),
                "gather_read_cold_us": round(float(np.median(gather_cold)),
                                             2),
                "output_write_cold_us": round(float(np.median(write_cold)),
                                              2),
                "note": "graph-timed medians over %d replays of 20 "
                        "calls; cold: MALL flushed before each call, the "
                        "write-back left after it charged" % ns,
            },
        },
    }
    variants = srows = None
    if not args.no_rows:
        variants = scale_variant_rows(torch, mxq, x, lay_out["src2dst"], R,
                                      H, q, B_sq, A, dev)
        srows = scatter_rows_row(torch, mxq, x, lay_out["src2dst"], R, H, q,
                                 T, K, A, dev)
    del q, s, out, outs

    if not args.no_rows:
        result["rows"] = other_rows(torch, mxq, si, dev,
                                    cpu=not args.no_cpu)
        result["rows"]["timing"] = ("each row: GPU time per call, 20 calls "
                                    "captured in a hipGraph, median and "
                                    "10-90 % spread over 100 replays; cold "
                                    "variants flush the MALL before each of "
                                    "100 eager calls; cpu_baseline: the "
                                    "oracle on this host's cores, median of "
                                    "3, and on one thread")
        result["rows"]["scale_variants"] = variants
        result["rows"]["scatter_rows"] = srows

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(torch, si, b, y, R, B_step,
                                              args.cpu_repeats)
    print(json.dumps(result), flush=True)


# ------------------------------------------- masked vs compact sweep

SWEEP_T = (256, 1024, 4096, 8192, 16384)
SWEEP_CASES = ((128, 128, "128 local experts, no expert parallelism"),
               (48, 384, "48 local experts of 384 (one GPU of eight)"))


def layout_sweep(torch, mxq, si, dev, H=7168, K=8):
    """Layout + scatter-quant + combine time per step under the masked and
    the compact layout, for each token count: the masked slab holds
    capacity T rows per local expert (the largest possible count, so any
    routing fits a static buffer); the compact buffer holds the static
    bound of the compact layout."""
    out = {"metric": "masked vs compact dispatch preprocessing time",
           "unit": "us", "hidden": H, "topk": K,
           "routing": "uniform top-8 over the global experts",
           "timing": "per call, 20 calls captured in a hipGraph, median "
                     "of 5 replays",
           "cases": []}
    for e_loc, e_glob, label in SWEEP_CASES:
        case = {"local_experts": e_loc, "global_experts": e_glob,
                "label": label, "points": []}
        for T in SWEEP_T:
            rng = np.random.default_rng(1000 * e_loc + T)
            ids_h = si.uniform_topk(rng, T, e_glob, K)
            ids = torch.from_numpy(ids_h).to(dev)
            w = torch.from_numpy(si.softmax_weights(rng, T, K)).to(dev)
            x = si.gaussian_bf16_device(T, (T, H), dev)
            local = int(((ids_h >= 0) & (ids_h < e_loc)).sum())
            pt = {"T": T, "local_assignments": local}
            for kind, cap in (("compact", 0), ("masked", T)):
                rows = (mxq.moe_compact_row_bound(T * K, e_loc, 128)
                        if kind == "compact" else e_loc * cap)
                lay = mxq.moe_layout(ids, 0, e_loc, kind, capacity=cap,
                                     num_rows=rows)
                q = torch.empty((rows, H), dtype=torch.uint8, device=dev)
                sc = torch.empty((rows, H // 128), dtype=torch.uint8,
                                 device=dev)
                y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
                y.view(torch.int16).fill_(0x3F80)
                o = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
                t_l = time_calls(torch, lambda: mxq.moe_layout(
                    ids, 0, e_loc, kind, capacity=cap, num_rows=rows,
                    out=lay), replays=10)
                t_s = time_calls(torch, lambda: mxq.moe_scatter_quant(
                    x, lay["src2dst"], rows, q=q, scales=sc), replays=10)
                t_c = time_calls(torch, lambda: mxq.moe_combine(
                    y, lay["src2dst"], w, out=o), replays=10)
                pt[kind] = {"rows": rows,
                            "buffer_gib": round(rows * H * 3 / 2 ** 30, 2),
                            "layout_us": round(t_l, 2),
                            "scatter_quant_us": round(t_s, 2),
                            "combine_us": round(t_c, 2),
                            "total_us": round(t_l + t_s + t_c, 2)}
                del lay, q, sc, y, o
            pt["compact_over_masked"] = round(
                pt["compact"]["total_us"] / pt["masked"]["total_us"], 4)
            case["points"].append(pt)
            del ids, w, x
        out["cases"].append(case)
    return out


# ------------------------------------------------- separately timed rows

def scale_variant_rows(torch, mxq, x, src2dst, R, H, q, B_sq, A, dev):
    """The prefill scatter under each exponent rule and scale placement,
    timed back to back (the plain entry point beside them, timed the same
    way)."""
    out = {"workload": "prefill scatter (8192 x 7168 -> 98048 rows, "
                       "UE8M0 group-128), back-to-back calls in a hipGraph "
                       "(the 117 MB of token rows stay in the MALL)",
           "algorithmic_bytes": B_sq}
    s_rows = torch.empty((R, H // 128), dtype=torch.uint8, device=dev)
    s_mn = mxq.packed_mn_scales(R, H // 128, dev)
    us = time_calls(torch, lambda: mxq.moe_scatter_quant(
        x, src2dst, R, "ue8m0_g128", q=q, scales=s_rows))
    out["moe_scatter_quant_us"] = round(us, 2)
    for rule in ("no_clip", "ocp_floor"):
        for layout, sc in (("rows", s_rows), ("packed_mn", s_mn)):
            us = time_calls(torch, lambda: mxq.moe_scatter_quant_ex(
                x, src2dst, R, "ue8m0_g128", rule, layout, q=q, scales=sc))
            out["%s/%s_us" % (rule, layout)] = round(us, 2)
            out["%s/%s_gbs" % (rule, layout)] = round(
                B_sq / (us * 1e-6) / 1e9, 2)
    # the block-scaled MFMA placement: one byte per 32-channel block, so
    # each group-128 scale is written four times (224 bytes per row)
    B_mfma = B_sq + A * (H // 32 - H // 128)
    out["mfma_algorithmic_bytes"] = B_mfma
    for layout in ("mfma32", "mfma16"):
        sc = mxq.mfma_scales(R, H, int(layout[4:]), dev)
        us = time_calls(torch, lambda: mxq.moe_scatter_quant_ex(
            x, src2dst, R, "ue8m0_g128", "no_clip", layout, q=q, scales=sc))
        out["no_clip/%s_us" % layout] = round(us, 2)
        out["no_clip/%s_gbs" % layout] = round(B_mfma / (us * 1e-6) / 1e9, 2)
    return out


def expanded_psum(counts, align):
    """psum of the expanded layout for per-expert counts: expert e starts at
    the aligned end of expert e - 1.  Returns (psum int32, aligned total)."""
    psum = np.zeros(len(counts), np.int32)
    prev = 0
    for e, c in enumerate(counts):
        psum[e] = -(-prev // align) * align + int(c)
        prev = int(psum[e])
    return psum, int(-(-prev // align) * align)


def psum_repack_prefill(torch, mxq, si, dev):
    """The two repack copies at a prefill-sized slab: 32 experts, capacity
    2048, counts uniform in [1024, 2048], 7168-wide rows."""
    E, MM, H = 32, 2048, 7168
    rng = np.random.default_rng(si.SEEDS["decode_masked"] + 7)
    cnt = rng.integers(1024, 2049, size=E)
    psum_h, total = expanded_psum(cnt, 128)
    psum = torch.from_numpy(psum_h).to(dev)
    xr = si.random_e4m3_bytes_device(si.SEEDS["fp8_dispatch"] + 1,
                                     (total, H), dev)
    xsc = torch.randint(100, 140, (total, H // 128), dtype=torch.uint8,
                        device=dev)
    slab = torch.empty((E * MM, H), dtype=torch.uint8, device=dev)
    slab_s = torch.empty((E * MM, H // 128), dtype=torch.uint8, device=dev)
    us_e = time_calls(torch, lambda: mxq.moe_expand_to_masked_slab(
        xr, psum, MM, 128, scales=xsc, slab=slab, slab_scales=slab_s))
    _, _, mm, _ = mxq.moe_expand_to_masked_slab(xr, psum, MM, 128, scales=xsc,
                                                 slab=slab, slab_scales=slab_s)
    del xr, xsc, slab, slab_s
    ys = si.gaussian_bf16_device(207, (E * MM, H), dev)
    w = torch.rand(total, device=dev)
    out = torch.empty((total, H), dtype=torch.bfloat16, device=dev)
    us_b = time_calls(torch, lambda: mxq.moe_masked_slab_to_expand(
        ys, mm, psum, MM, 128, weights=w, out=out))
    real = int(cnt.sum())
    b_e = real * 2 * (H + H // 128) + E * 8
    b_b = real * (2 * H * 2 + 4)
    return {"workload": "%d real rows in %d (32 experts, 128-aligned) <-> "
                        "slab [32, 2048, 7168]" % (real, total),
            "expand_to_masked_slab_us": round(us_e, 2),
            "expand_bytes": b_e,
            "expand_gbs": round(b_e / (us_e * 1e-6) / 1e9, 2),
            "masked_slab_to_expand_us": round(us_b, 2),
            "slab_to_expand_bytes": b_b,
            "slab_to_expand_gbs": round(b_b / (us_b * 1e-6) / 1e9, 2)}


def scatter_rows_row(torch, mxq, x, src2dst, R, H, q, T, K, A, dev):
    """The psum prefill path: the same tokens already quantized by the
    sender (fp8 rows + 56 UE8M0 bytes) copied into the compact layout."""
    q_tok, s_tok = mxq.mx_quant_live_rows(
        x, 1, torch.tensor([T], dtype=torch.int32, device=dev),
        fmt="ue8m0_g128")
    so = torch.empty((R, H // 128), dtype=torch.uint8, device=dev)
    us = time_calls(torch, lambda: mxq.moe_scatter_rows(
        q_tok, src2dst, R, scales=s_tok, out=q, out_scales=so))
    byts = T * (H + H // 128) + A * (H + H // 128) + T * K * 4
    return {"workload": "prefill: 8192 fp8 token rows + 56 UE8M0 bytes "
                        "-> 65536 rows of the 98048-row compact layout",
            "us": round(us, 2), "algorithmic_bytes": byts,
            "gbs": round(byts / (us * 1e-6) / 1e9, 2)}


def cpu_row(fn, nbytes=None, units=None, unit_name=None, repeats=3,
            cpu=True):
    """The oracle timed on this host's cores beside a GPU row: wall clock,
    median of `repeats` runs on every OpenMP thread, then one run on one
    thread.  Returns None when the CPU leg is off."""
    if not cpu:
        return None
    import oracle
    cores = oracle.max_threads()
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        fn()
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(cores)
    r = {"kind": "oracle", "cores": cores, "seconds": round(t, 5),
         "single_thread_seconds": round(t1, 5)}
    if nbytes is not None:
        r["gbs"] = round(nbytes / t / 1e9, 4)
        r["single_thread_gbs"] = round(nbytes / t1 / 1e9, 4)
    if units is not None:
        r[unit_name + "_per_s"] = round(units / t, 1)
        r["single_thread_" + unit_name + "_per_s"] = round(units / t1, 1)
    return r


def other_rows(torch, mxq, si, dev, cpu=True):
    import_oracle = cpu
    if import_oracle:
        import oracle
    rows = {}
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    # masked decode slab: one GPU's 32 of 256 experts, T=128
    d = si.decode_masked()
    ids = torch.from_numpy(d.topk_ids).to(dev)
    x = torch.from_numpy(d.x.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(d.topk_weights).to(dev)
    R = 32 * 128
    q = torch.empty((R, d.H), dtype=torch.uint8, device=dev)
    s = torch.empty((R, d.H // 128), dtype=torch.uint8, device=dev)
    yv = si.gaussian_bf16_device(202, (R, d.H), dev)
    lay = mxq.moe_layout(ids, 0, 32, "masked", capacity=128)
    loc_mask = (d.topk_ids >= 0) & (d.topk_ids < 32)
    loc = int(loc_mask.sum())
    touched_d = int(loc_mask.any(axis=1).sum())
    b_sq_d = bytes_scatter(touched_d, d.T, d.K, d.H, 128, loc)
    b_cb_d = bytes_combine(d.T, d.K, d.H, loc)
    r_l = timed_row(torch, lambda: mxq.moe_layout(
        ids, 0, 32, "masked", capacity=128, out=lay))
    r_s = timed_row(torch, lambda: mxq.moe_scatter_quant(
        x, lay["src2dst"], R, q=q, scales=s))
    r_c = timed_row(torch, lambda: mxq.moe_combine(yv, lay["src2dst"], w))

    def layout_then_scatter():
        mxq.moe_layout(ids, 0, 32, "masked", capacity=128, out=lay)
        mxq.moe_scatter_quant(x, lay["src2dst"], R, q=q, scales=s)
    r_ls = timed_row(torch, layout_then_scatter)
    r_f = timed_row(torch, lambda: mxq.moe_layout_scatter_quant(
        ids, x, 0, 32, "masked", capacity=128, out=lay, q=q, scales=s))
    us_l, us_s, us_c, us_f = r_l["us"], r_s["us"], r_c["us"], r_f["us"]
    rows["decode_masked"] = {
        "workload": "T=128, hidden 7168, experts [0,32) of 256 local, top-8, "
                    "slab capacity 128, UE8M0 group-128",
        "local_assignments": loc, "layout_us": us_l,
        "scatter_quant_us": us_s, "combine_us": us_c,
        "layout_then_scatter_quant_us": r_ls["us"],
        "fused_layout_scatter_quant_us": us_f,
        "us_spread": {"layout": r_l["us_spread"],
                      "scatter_quant": r_s["us_spread"],
                      "combine": r_c["us_spread"],
                      "fused_layout_scatter_quant": r_f["us_spread"]},
        "assignments_per_s": round(loc / ((us_l + us_s + us_c) * 1e-6), 1),
        "assignments_per_s_fused": round(loc / ((us_f + us_c) * 1e-6), 1),
        "scatter_quant_bytes": b_sq_d, "combine_bytes": b_cb_d,
        "note": "latency-bound: %.2f MB and %.2f MB move in the scatter and "
                "the combine" % (b_sq_d / 1e6, b_cb_d / 1e6)}
    if cpu:
        yv_h = yv.view(torch.int16).cpu().numpy().view(np.uint16)

        def ora_decode():
            ol = oracle.moe_layout(d.topk_ids, 0, 32, "masked",
                                   capacity=128)
            oracle.scatter_quant(d.x, ol["src2dst"], 128, R)
            oracle.combine(yv_h, ol["src2dst"], d.topk_weights)
        rows["decode_masked"]["cpu_baseline"] = cpu_row(
            ora_decode, nbytes=b_sq_d + b_cb_d, units=loc,
            unit_name="assignments")
        rows["decode_masked"]["cpu_baseline"]["sample"] = (
            "the whole decode batch: layout + scatter_quant + combine")

    # send-side MX quant over live rows: 24576 x 7168 padded, 112 live
    xs = si.gaussian_bf16_device(404, (24576, 7168), dev)
    qs = torch.empty((24576, 7168), dtype=torch.uint8, device=dev)
    ss = torch.empty((24576, 224), dtype=torch.uint8, device=dev)
    res = {}
    xs_h = xs.view(torch.int16).cpu().numpy().view(np.uint16) if cpu else None
    qs_h = np.zeros((24576, 7168), np.uint8) if cpu else None
    ss_h = np.zeros((24576, 224), np.uint8) if cpu else None
    for name, live in (("14x8", [14] * 8), ("112+0x7", [112] + [0] * 7),
                       ("empty", [0] * 8)):
        lc = torch.tensor(live, dtype=torch.int32, device=dev)
        n = sum(live)
        byts = n * (7168 * 2 + 7168 + 224) + 32
        res[name] = dict(live_rows=n, **timed_row(
            torch, lambda: mxq.mx_quant_live_rows(xs, 8, lc, q=qs, scales=ss),
            nbytes=byts, units=n, unit_name="rows"))
        if cpu:
            live_h = np.asarray(live, np.int32)
            res[name]["cpu_baseline"] = cpu_row(
                lambda: oracle.mx_quant_live_rows(xs_h, 8, live_h, 32,
                                                  qs_h, ss_h),
                nbytes=byts, units=n, unit_name="rows")
            res[name]["cpu_baseline"]["sample"] = "the same %d live rows" % n
    res["padded_grid_equivalent_bytes"] = 24576 * (7168 * 2 + 7168 + 224)
    # the same quant over every row of the padded buffer (what a receiver
    # that sizes its grid by the buffer pays)
    lc = torch.full((8,), 3072, dtype=torch.int32, device=dev)
    pad = timed_row(torch, lambda: mxq.mx_quant_live_rows(
        xs, 8, lc, q=qs, scales=ss), reps=5)
    res["padded_grid_us"] = pad["us"]
    res["padded_grid_us_spread"] = pad["us_spread"]
    res["padded_over_live_14x8"] = round(pad["us"] / res["14x8"]["us"], 1)
    # the same 14x8 live rows with the scales in the block-scaled MFMA
    # placement (32-row tiles)
    lc = torch.tensor([14] * 8, dtype=torch.int32, device=dev)
    sm = mxq.mfma_scales(24576, 7168, 32, dev)
    us = time_calls(torch, lambda: mxq.mx_quant_live_rows_ex(
        xs, 8, lc, "e8m0_g32", scale_layout="mfma32", q=qs, scales=sm))
    res["14x8_mfma32_us"] = round(us, 2)
    # an empty kernel launched the same way: what one launch costs here
    res["note"] = ("a launch costs about 2.1 us per call in this timing "
                   "(measured with an empty kernel), the floor of the "
                   "empty batch")
    res["workload"] = ("24576 x 7168 bf16 padded buffer = 8 segments of "
                       "3072 rows, e8m0 group-32 (224 scales/row)")
    rows["live_rows_mx"] = res
    del xs, qs, ss, xs_h, qs_h, ss_h

    # per-token -> per-tensor requant, 16384 x 4096
    rb = si.requant_input()
    qi = torch.from_numpy(rb.q).to(dev)
    sc = torch.from_numpy(rb.scales).to(dev)
    qo = torch.empty_like(qi)
    Sd = torch.empty(1, dtype=torch.float32, device=dev)
    rws = torch.empty(mxq.requant_workspace_bytes(*qi.shape),
                      dtype=torch.uint8, device=dev)
    byts = 2 * qi.numel() + qi.shape[0] * 4 + 4
    rq = timed_row(torch, lambda: mxq.requant_per_token_to_per_tensor(
        qi, sc, q_out=qo, tensor_scale=Sd, workspace=rws), nbytes=byts,
        flush=flush)
    # every token scale equal (2^-3): every row's bound is the largest
    sc_eq = torch.full_like(sc, 2.0 ** -3)
    rq_eq = timed_row(torch, lambda: mxq.requant_per_token_to_per_tensor(
        qi, sc_eq, q_out=qo, tensor_scale=Sd, workspace=rws), nbytes=byts)
    # the max pass's worst case: equal scales and no row holding +-448 (the
    # 448 bytes lowered to 416), so no row attains the common bound and
    # every row must be read
    qi_low = torch.where((qi & 0x7F) == 0x7E, qi - 1, qi)
    rq_wc = timed_row(torch, lambda: mxq.requant_per_token_to_per_tensor(
        qi_low, sc_eq, q_out=qo, tensor_scale=Sd, workspace=rws),
        nbytes=byts)
    del qi_low
    rows["requant"] = {"workload": "16384 x 4096 fp8, per-token scales "
                                   "2^U, U~U[-8,4]", **rq,
                       "equal_scales_us": rq_eq["us"],
                       "equal_scales_gbs": rq_eq["gbs"],
                       "equal_scales_us_spread": rq_eq["us_spread"],
                       "equal_scales_no_row_at_448_us": rq_wc["us"],
                       "equal_scales_no_row_at_448_gbs": rq_wc["gbs"],
                       "note": "warm: the 64 MiB input stays in the 256 MB "
                               "MALL across the two passes and back-to-back "
                               "calls; cold: MALL flushed by reading 512 MB "
                               "before each call, the write-back left after "
                               "it charged; equal_scales: every token "
                               "scale 2^-3, so every row's bound is the "
                               "largest (rows holding 448 settle the max "
                               "pass at once) (warm); equal_scales_no_row_"
                               "at_448: the same with no byte at +-448, so "
                               "the max pass reads every row (warm)"}
    if cpu:
        rows["requant"]["cpu_baseline"] = cpu_row(
            lambda: oracle.requant_per_token_to_per_tensor(rb.q, rb.scales),
            nbytes=byts, units=qi.shape[0], unit_name="rows")
        rows["requant"]["cpu_baseline"]["sample"] = "the whole 16384 x 4096"
    del qi, qo

    # psum (expanded) layout repack at the decode shape: the dispatcher's
    # expanded rows (counts of the decode routing, 128-aligned) -> masked
    # slab [32, 128, 7168] fp8 + 56 UE8M0 bytes, and the bf16 slab back to
    # expanded rows with the top-k weights applied
    counts = mxq.moe_layout(ids, 0, 32, "masked", capacity=128)["counts"]
    cnt = counts.cpu().numpy().astype(np.int64)
    psum_h, total = expanded_psum(cnt, 128)
    psum = torch.from_numpy(psum_h).to(dev)
    xr = torch.randint(0, 255, (total, 7168), dtype=torch.uint8, device=dev)
    xsc = torch.randint(100, 140, (total, 56), dtype=torch.uint8, device=dev)
    slab = torch.empty((32 * 128, 7168), dtype=torch.uint8, device=dev)
    slab_s = torch.empty((32 * 128, 56), dtype=torch.uint8, device=dev)
    real = int(cnt.sum())
    r_e = timed_row(torch, lambda: mxq.moe_expand_to_masked_slab(
        xr, psum, 128, 128, scales=xsc, slab=slab, slab_scales=slab_s))
    _, _, mm, _ = mxq.moe_expand_to_masked_slab(xr, psum, 128, 128,
                                                 scales=xsc, slab=slab,
                                                 slab_scales=slab_s)
    ys = si.gaussian_bf16_device(206, (32 * 128, 7168), dev)
    wexp = torch.rand(total, device=dev)
    oexp = torch.zeros((total, 7168), dtype=torch.bfloat16, device=dev)
    r_b = timed_row(torch, lambda: mxq.moe_masked_slab_to_expand(
        ys, mm, psum, 128, 128, weights=wexp, out=oexp))
    us_m = time_calls(torch, lambda: mxq.moe_m_indices_from_psum(
        psum, total, 128))
    rows["psum_repack"] = {
        "workload": "decode expanded layout: %d real rows in %d (32 experts, "
                    "128-aligned) <-> slab [32, 128, 7168]" % (real, total),
        "expand_to_masked_slab_us": r_e["us"],
        "expand_to_masked_slab_us_spread": r_e["us_spread"],
        "expand_bytes": real * 2 * (7168 + 56) + 32 * 8,
        "masked_slab_to_expand_us": r_b["us"],
        "masked_slab_to_expand_us_spread": r_b["us_spread"],
        "slab_to_expand_bytes": real * (2 * 7168 * 2 + 4),
        "m_indices_from_psum_us": round(us_m, 2)}
    del xr, xsc, slab, slab_s, ys, oexp
    rows["psum_repack"]["prefill_shape"] = psum_repack_prefill(torch, mxq, si,
                                                               dev)

    # receive-side upscale: fp8 + group-128 fp32 scales -> bf16 over the
    # live rows of the 3072 x 8 padded receive buffer
    rows_u, H_u, n_u = 24576, 7168, 8192
    qu = si.random_e4m3_bytes_device(si.SEEDS["fp8_dispatch"], (rows_u, H_u),
                                     dev)
    su = torch.from_numpy(si.group_scales_f32(
        np.random.default_rng(si.SEEDS["fp8_dispatch"]),
        (rows_u, H_u // 128))).to(dev)
    ou = torch.empty((rows_u, H_u), dtype=torch.bfloat16, device=dev)
    byts = n_u * (H_u + 4 * (H_u // 128) + 2 * H_u)
    up = timed_row(torch, lambda: mxq.upscale_fp8_to_bf16(qu, su, n_u,
                                                         out=ou),
                   nbytes=byts)
    # the same calls writing three output buffers in turn (3 x 117 MB, more
    # than the 256 MB MALL), so each call's output reaches HBM during the
    # following calls instead of being overwritten in the cache
    ous = [ou] + [torch.empty_like(ou) for _ in range(2)]
    turn = [0]

    def up_rot():
        turn[0] += 1
        mxq.upscale_fp8_to_bf16(qu, su, n_u, out=ous[turn[0] % 3])
    us_rot = time_calls(torch, up_rot, reps=21)
    rows["upscale"] = {
        "workload": "24576 x 7168 fp8 receive buffer, group-128 fp32 scales, "
                    "first 8192 rows upscaled to bf16", **up,
        "rotating_outputs_us": round(us_rot, 2),
        "rotating_outputs_gbs": round(byts / (us_rot * 1e-6) / 1e9, 2)}
    del qu, su, ou, ous

    # weight-side UE8M0 block requant of 32 local experts' gate/up and down
    # weights (load time)
    wr = {"workload": "32 experts: gate/up [32, 4096, 7168] and down "
                      "[32, 7168, 2048] e4m3 with 128 x 128 fp32 block "
                      "scales -> UE8M0 block scales"}
    for name, shape in (("gate_up", (32, 4096, 7168)),
                        ("down", (32, 7168, 2048))):
        qw = si.random_e4m3_bytes_device(si.SEEDS["block_weights"], shape,
                                         dev)
        B_, N_, K_ = shape
        sw = torch.from_numpy(si.group_scales_f32(
            np.random.default_rng(si.SEEDS["block_weights"]),
            (B_, N_ // 128, K_ // 128), 2.0 ** -16, 2.0 ** -8)).to(dev)
        qo = torch.empty_like(qw)
        so = torch.empty(sw.shape, dtype=torch.uint8, device=dev)
        nblk = B_ * (N_ // 128) * (K_ // 128)
        wr[name] = timed_row(torch, lambda: mxq.requant_weight_block_ue8m0(
            qw, sw, q_out=qo, scales_out=so), nbytes=2 * qw.numel() + 5 * nblk,
            reps=10)
        del qw, sw, qo, so
    rows["weight_requant"] = wr

    # large combine: 16384 tokens x 4096 from 147328 rows, top-8 of 128
    cids, cw = si.large_combine_routing()
    idsd = torch.from_numpy(cids).to(dev)
    lay = mxq.moe_layout(idsd, 0, 128, "compact")
    yl = si.gaussian_bf16_device(505, (lay["num_rows"], 4096), dev)
    wd = torch.from_numpy(cw).to(dev)
    ols = [torch.empty((16384, 4096), dtype=torch.bfloat16, device=dev)
           for _ in range(N_OUT)]
    nxt = rotation(ols)
    byts = bytes_combine(16384, 8, 4096, 16384 * 8)
    rows["large_combine"] = {
        "workload": "T=16384, hidden 4096, 128 experts top-8, 147328-row "
                    "layout",
        **timed_row(torch, lambda: mxq.moe_combine(yl, lay["src2dst"], wd,
                                                   out=nxt()),
                    nbytes=byts, flush=flush)}
    if cpu:
        yl_h = yl.view(torch.int16).cpu().numpy().view(np.uint16)
        s2d_h = lay["src2dst"].cpu().numpy()
        rows["large_combine"]["cpu_baseline"] = cpu_row(
            lambda: oracle.combine(yl_h, s2d_h, cw), nbytes=byts,
            units=16384, unit_name="tokens")
        rows["large_combine"]["cpu_baseline"]["sample"] = (
            "the whole combine (131072 rows -> 16384 tokens)")
        del yl_h
    del flush
    return rows


# ------------------------------------------------------- CPU oracle leg

def cpu_baseline(torch, si, b, y_dev, R, B_step, repeats):
    """The CPU oracle, as it stands, on the same prefill workload: layout,
    scatter+quant and combine over all 8192 tokens, median of `repeats`."""
    import oracle
    y_host = y_dev.view(torch.int16).cpu().numpy().view(np.uint16)
    cores = oracle.max_threads()
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        lay = oracle.moe_layout(b.topk_ids, 0, b.n_local, "compact")
        oracle.scatter_quant(b.x, lay["src2dst"], b.group, R)
        oracle.combine(y_host, lay["src2dst"], b.topk_weights)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    # the same work on one thread, once
    oracle.set_threads(1)
    t0 = time.perf_counter()
    lay = oracle.moe_layout(b.topk_ids, 0, b.n_local, "compact")
    oracle.scatter_quant(b.x, lay["src2dst"], b.group, R)
    oracle.combine(y_host, lay["src2dst"], b.topk_weights)
    t1 = time.perf_counter() - t0
    oracle.set_threads(cores)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(B_step / t / 1e9, 3), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": "the full prefill workload (8192 tokens, 65536 "
                      "assignments): layout + scatter_quant + combine, "
                      "median of %d runs, %.2f s each" % (repeats, t),
            "single_thread": {"value": round(B_step / t1 / 1e9, 3),
                              "seconds": round(t1, 2)},
            "cpu_model": cpu_model}


if __name__ == "__main__":
    main()
