#!/usr/bin/env python3
"""Benchmark of the HiLS attention hot path on one MI355X.

Headline: the 1.4B-shape long prefill forward (batch 1, 32 query / 8 KV
heads, d 128, 131072 tokens, chunk 64, top-16, 1024-token window, Q-Cal rank
32 from hidden 2048, a planted needle chunk every 16384 tokens), bf16, seeded
synthetic inputs resident in HBM. One step = one hils_attn_fwd call: Q-Cal,
routing (scores + GQA max + top-K), window and selected-chunk attention,
fusion.

Prints ONE JSON line: prefill tokens/s; the time, algorithmic flops and MFMA
fraction of every launch step (HIP events recorded by the library around each
step of every timed call); the roofline of the longest single launch; the
chunk phase, the window phase and both together; and the fp64 CPU oracle
timed on every host core the process may use (one process per core, run
before the GPU is touched) on a bounded sample of the same workload. Extra
legs in the same line:
  prefill_345m      the 345M-shape prefill (B4, H16, d64, 8192 tokens), with
                    the chunk-major phase split of the same problem;
  prefill_512k      the 524288-token prefill of the 345M shape with top-32
                    (the paper's long-context measurement setup);
  decode            the 512K-context decode step of 32 sequences (µs per
                    step against the HBM roofline, cold last-level cache;
                    also from a HIP graph and over a paged cache) with the
                    4M-token single-sequence decode as "long_context", each
                    with its oracle baseline;
  train             forward + backward tokens/s and MFMA fraction, with its
                    oracle baseline;
  landmark, hope    the landmark summary and the HoPE rotation against HBM;
  packing           chunk-id overlap of adjacent queries and the three
                    forward strategies on independent and on
                    position-correlated queries.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HiLS prefill tokens/s + decode µs/step at 512K; % of HBM / bf16 MFMA peak"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
HOST_CORE_SHARE = 16             # host cores that go with one GPU on the measurement machine


# --------------------------------------------------------------------------
# algorithmic work (what the method has to do, independent of the kernels)
# --------------------------------------------------------------------------
def n_distant(i, W, S):
    return max(0, (i - W + 1) // S)


def _positions(wl):
    import numpy as np
    i = np.arange(wl.N, dtype=np.int64)
    nd = np.maximum(0, (i - wl.W + 1) // wl.S)
    return i, nd


def fwd_algorithmic_flops(wl):
    """Flops of the attention: 4*d per (query head, attended token), over the
    window [nd*S, i] and over the selected chunks (returned separately)."""
    i, nd = _positions(wl)
    win = int((i + 1 - nd * wl.S).sum())
    chk = int((nd.clip(max=wl.K) * wl.S).sum())
    rows = wl.B * wl.Hq
    return rows * 4 * wl.d * win, rows * 4 * wl.d * chk


def route_algorithmic_flops(wl):
    """2*d per (query head, distant chunk): the O(N^2/S) scoring term."""
    _, nd = _positions(wl)
    return wl.B * wl.Hq * 2 * wl.d * int(nd.sum())


def qcal_algorithmic_flops(wl):
    return wl.B * wl.N * wl.Hq * (2 * wl.r * wl.D + 2 * wl.d * wl.r) if wl.r else 0


def train_algorithmic_flops(wl):
    """Forward 4*d and backward 10*d flops per (query head, attended token)
    (backward: S, dP, dq, dk and dv products), plus the routing scores."""
    win_f, chk_f = fwd_algorithmic_flops(wl)
    attn = win_f + chk_f
    return attn + attn * 10 // 4 + route_algorithmic_flops(wl)


def decode_bytes(wl):
    """Algorithmic HBM bytes of one decode step: every distant landmark key and
    bias, the K selected chunks and the window, K and V, per (sequence, KV head)."""
    el = 2 if wl.dtype == "bf16" else 4
    tot = 0
    for n in ([wl.N] * wl.B if wl.seq_len is None else wl.seq_len):
        i = n - 1
        nd = n_distant(i, wl.W, wl.S)
        toks = min(wl.K, nd) * wl.S + (i + 1 - nd * wl.S)
        tot += wl.Hkv * (nd * (wl.d * el + el) + toks * 2 * wl.d * el)
    return tot


def landmark_bytes(wl):
    """HBM bytes the landmark summary has to move per call: the forward reads
    the keys and landmark queries and writes kL, e; the backward reads the
    keys, queries, dkL and de, writes dqL and reads and writes the fp32 dk it
    adds into."""
    bg, C, d = wl.B * wl.Hkv, wl.N // wl.S, wl.d
    el = 2 if wl.dtype == "bf16" else 4
    keys = bg * C * wl.S * d
    fwd = keys * el + bg * C * d * el * 2 + bg * C * el
    bwd = keys * el + bg * C * d * el + bg * C * (d + 1) * 4 + bg * C * d * 4 + 2 * keys * 4
    return fwd, bwd


# --------------------------------------------------------------------------
# HBM traffic of a kernel from its committed rocprofv3 counter summary
# --------------------------------------------------------------------------
CSRC = os.path.join(ROOT, "learnable_chunk_sparse_amd", "csrc")
# (kernel step, workload) -> (summary file, the sources the counters were taken on)
TRAFFIC = {
    ("window", "prefill_1p4b"): ("fwd_cm_window__prefill_1p4b__hbm_traffic.md",
                                 ["attn_fwd_cm.hip", "hils_common.h"]),
    ("chunks", "prefill_1p4b"): ("fwd_cm_chunks__prefill_1p4b__hbm_traffic.md",
                                 ["attn_fwd_cm.hip", "hils_common.h"]),
    ("window", "prefill_345m"): ("attn_fwd__prefill_345m__hbm_traffic.md",
                                 ["attn_fwd.hip", "attn_fwd_sparse.hip", "hils_common.h"]),
    ("route", "prefill_345m_512k"): ("route__prefill_345m_512k__hbm_traffic.md",
                                     ["route.hip", "hils_common.h"]),
    # decode: the whole step (its four launches) per call
    ("decode", "decode_7b_512k"): ("decode__decode_7b_512k__hbm_traffic.md",
                                   ["decode.hip", "hils_common.h"]),
    ("decode", "decode_4m"): ("decode__decode_4m__hbm_traffic.md", ["decode.hip", "hils_common.h"]),
}


def sources_digest(names):
    """sha256 over kernel source files (counters only hold for the kernel
    they were taken on)."""
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(step, workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    calibration) from the committed counter summary of that kernel and
    workload, or None when there is none or it was taken on other sources."""
    entry = TRAFFIC.get((step, workload))
    if entry is None:
        return None
    try:
        fields = {}
        with open(os.path.join(ROOT, "profiles", entry[0])) as f:
            for line in f:
                if line.startswith("- ") and ":" in line:
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("sources_sha256") != sources_digest(entry[1]):
            return None
        return float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# --------------------------------------------------------------------------
# the fp64 oracle on the host cores (forked before anything touches the GPU)
# --------------------------------------------------------------------------
def host_cores():
    """(worker processes to use, cores visible to this process)."""
    visible = len(os.sched_getaffinity(0))
    return max(1, min(visible, HOST_CORE_SHARE)), visible


def _f64_inputs(t):
    """Inputs converted once to fp64 NumPy (the oracle then reads them in
    place, as the GPU reads its inputs already resident in HBM)."""
    from oracle import hils_oracle as H
    return {k: (v if k == "seq_len" else H.f64(v)) for k, v in t.items()}


def _prep_prefill(wl_name, b, g, rows):
    from workloads import WORKLOADS, make_group_inputs
    from oracle import hils_oracle as H
    wl = WORKLOADS[wl_name]
    t = _f64_inputs(make_group_inputs(wl, b, g, h_rows=rows if wl.r else None))

    def run():
        H.hils_forward(t, wl.S, wl.K, wl.W, rows=rows)
        return len(rows)
    return run


def _prep_decode(wl_name, b, g):
    from workloads import WORKLOADS, make_group_inputs
    from oracle import hils_oracle as H
    wl = WORKLOADS[wl_name]
    # the cache rows the step reads (its selection and window); the rest stay
    # NaN, which the oracle never touches
    t0 = make_group_inputs(wl, b, g, kv_rows=[])
    n = int(t0["seq_len"][0])
    sel = H.hils_decode(t0, wl.S, wl.K, wl.W, rank_only=True)["topk"][0, 0]
    nd = n_distant(n - 1, wl.W, wl.S)
    rows = [c * wl.S + j for c in sel.tolist() if c >= 0 for j in range(wl.S)]
    rows += list(range(nd * wl.S, n))
    del t0
    t = _f64_inputs(make_group_inputs(wl, b, g, kv_rows=rows))

    def run():
        H.hils_decode(t, wl.S, wl.K, wl.W)
        return 1
    return run


def _prep_train(wl_name, b, g):
    from workloads import WORKLOADS, make_group_inputs
    from oracle import hils_oracle as H
    wl = WORKLOADS[wl_name]
    t = _f64_inputs(make_group_inputs(wl, b, g))

    def run():
        H.hils_backward(t, t["dO"], wl.S, wl.K, wl.W)
        return 1
    return run


_PREP = {"prefill": _prep_prefill, "decode": _prep_decode, "train": _prep_train}


# seconds a worker keeps repeating its units (short units, e.g. one decode step)
_MIN_SECONDS = {"prefill": 0.0, "decode": 2.0, "train": 0.0}


def _cpu_worker(j, kind, tasks, barrier, out):
    """One single-threaded process: prepare its units (inputs generated and
    converted, not timed), wait for every worker, then run them back to back
    (again and again until _MIN_SECONDS[kind] have passed)."""
    try:
        import torch
        torch.set_num_threads(1)
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            runs = [_PREP[kind](*a) for a in tasks]
            barrier.wait()
            t0 = time.perf_counter()
            units = 0
            while True:
                units += sum(r() for r in runs)
                t1 = time.perf_counter()
                if t1 - t0 >= _MIN_SECONDS[kind]:
                    break
        out.put((j, units, t0, t1, None))
    except BaseException as ex:  # report instead of leaving the parent waiting
        try:
            barrier.abort()
        except Exception:
            pass
        out.put((j, 0, 0.0, 0.0, f"{type(ex).__name__}: {ex}"))


def run_oracle_workers(kind, tasks_per_worker, timeout_s=900.0):
    """Fork one process per task list; returns (units done, wall seconds from
    the common start to the last finish, processes)."""
    import multiprocessing as mp
    import queue
    ctx = mp.get_context("fork")
    nw = len(tasks_per_worker)
    barrier = ctx.Barrier(nw, timeout=timeout_s)
    out = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(j, kind, tl, barrier, out), daemon=True)
             for j, tl in enumerate(tasks_per_worker)]
    for p in procs:
        p.start()
    res = []
    deadline = time.time() + timeout_s
    try:
        while len(res) < nw:
            try:
                res.append(out.get(timeout=5.0))
            except queue.Empty:
                if time.time() > deadline:
                    raise RuntimeError(f"oracle workers ({kind}) did not finish in {timeout_s:.0f} s")
                dead = [p for p in procs if p.exitcode not in (None, 0)]
                if dead:
                    raise RuntimeError(f"an oracle worker ({kind}) exited with {dead[0].exitcode}")
    finally:
        for p in procs:
            p.join(timeout=10.0)
            if p.is_alive():
                p.kill()
                p.join()
    errs = [r[4] for r in res if r[4]]
    if errs:
        raise RuntimeError(f"oracle worker ({kind}) failed: {errs[0]}")
    units = sum(r[1] for r in res)
    wall = max(r[3] for r in res) - min(r[2] for r in res)
    return units, wall, nw


def _deal(tasks, nw):
    """Round-robin the tasks over at most nw workers (no empty worker)."""
    nw = max(1, min(nw, len(tasks)))
    return [tasks[j::nw] for j in range(nw)]


def _baseline(value, unit, nw, visible, sample, higher=True):
    return {"value": value, "unit": unit, "cores": nw, "kind": "oracle",
            "higher_is_better": higher, "visible_cores": visible, "blas_threads_per_process": 1,
            "sample": sample}


def cpu_baseline_prefill(wl, npos):
    """npos evenly spaced query positions of every (batch, KV group), split
    over the workers; tokens/s of the whole workload (a token costs B*Hkv
    group-rows, each covering its G query heads)."""
    nw, visible = host_cores()
    pos = [(j + 1) * wl.N // npos - 1 for j in range(npos)]
    pairs = [(b, g) for b in range(wl.B) for g in range(wl.Hkv)]
    m = max(1, nw // len(pairs))
    tasks = [(wl.name, b, g, pos[k::m]) for (b, g) in pairs for k in range(m)]
    units, wall, used = run_oracle_workers("prefill", _deal(tasks, nw))
    tok_s = units / wall / (wl.B * wl.Hkv) * wl.B
    return _baseline(tok_s, "tokens/s", used, visible,
                     f"{npos} evenly spaced query positions x {wl.B * wl.Hkv} (batch, KV head) "
                     f"slabs = {units} group-rows of {wl.G} heads in {wall:.1f} s on {used} "
                     f"single-threaded processes, scaled by {wl.N}/{npos} positions")


def cpu_baseline_decode(wl, nseq):
    """The first nseq sequences, every KV group: microseconds per step of
    the whole batch (all B*Hkv (sequence, KV group) units)."""
    nw, visible = host_cores()
    tasks = [(wl.name, b, g) for b in range(min(nseq, wl.B)) for g in range(wl.Hkv)]
    units, wall, used = run_oracle_workers("decode", _deal(tasks, nw))
    us = wall * (wl.B * wl.Hkv / units) * 1e6
    return _baseline(us, "µs/step", used, visible,
                     f"{len(tasks)} of {wl.B * wl.Hkv} (sequence, KV head) units, each run "
                     f"repeatedly: {units} unit steps in {wall:.1f} s on {used} single-threaded "
                     f"processes, scaled by {wl.B * wl.Hkv} units per step", higher=False)


def cpu_baseline_train(wl, ngroups):
    """Forward + backward of whole (batch 0, KV group) slabs: tokens/s of the
    whole batch."""
    nw, visible = host_cores()
    tasks = [(wl.name, 0, g) for g in range(min(ngroups, wl.Hkv))]
    units, wall, used = run_oracle_workers("train", _deal(tasks, nw))
    step_s = wall * (wl.B * wl.Hkv / units)
    return _baseline(wl.B * wl.N / step_s, "tokens/s", used, visible,
                     f"forward + backward of {units} of {wl.B * wl.Hkv} whole (batch, KV head) "
                     f"slabs in {wall:.1f} s on {used} single-threaded processes, scaled by "
                     f"{wl.B * wl.Hkv}/{units}")


def cpu_baselines(args, legs):
    """Every oracle leg (before the GPU is touched: the workers are forked)."""
    from workloads import WORKLOADS
    out = {}

    def leg(name, fn):
        t0 = time.perf_counter()
        try:
            out[name] = fn()
        except Exception as ex:  # a failed baseline is reported, not fatal
            out[name] = {"error": str(ex)}
        print(json.dumps({"cpu_baseline": name, "seconds": round(time.perf_counter() - t0, 1)}),
              file=sys.stderr, flush=True)

    leg("prefill", lambda: cpu_baseline_prefill(WORKLOADS[args.workload], args.cpu_positions))
    if "decode" in legs:
        leg("decode", lambda: cpu_baseline_decode(WORKLOADS[args.decode_workload], 2))
        if "decode_long" in legs:
            leg("decode_long", lambda: _decode_long_baseline(WORKLOADS["decode_4m"]))
    if "train" in legs:
        leg("train", lambda: cpu_baseline_train(WORKLOADS["train_345m"], 16))
    return out


def _decode_long_baseline(wl):
    """The 4M-token decode on every other KV head (the fp64 cache of one
    head is 4.3 GB): microseconds per step of all heads."""
    nw, visible = host_cores()
    tasks = [(wl.name, 0, g) for g in range(0, wl.Hkv, 2)]
    units, wall, used = run_oracle_workers("decode", _deal(tasks, nw))
    us = wall * (wl.B * wl.Hkv / units) * 1e6
    return _baseline(us, "µs/step", used, visible,
                     f"{len(tasks)} of {wl.Hkv} KV heads (every other), each run repeatedly: "
                     f"{units} unit steps in {wall:.1f} s on {used} single-threaded processes, "
                     f"scaled by {wl.Hkv} units per step", higher=False)


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------
def profile_sample(torch, L, workload="prefill_1p4b"):
    """A short fixed run for rocprofv3 counter passes: three prefill forwards
    (or decode steps) of the workload, then the calibration copy (1 GiB fp32
    read, 1 GiB written) whose FETCH_SIZE / WRITE_SIZE scale the kernel's
    counters."""
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[workload]
    t = make_inputs(wl, device="cuda")
    if wl.mode == "decode":
        bufs = L.decode_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))
        for _ in range(3):
            L.hils_decode(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                          seq_len=t["seq_len"], h=t.get("h"), W_down=t.get("W_down"),
                          W_up=t.get("W_up"), out=bufs)
    else:
        bufs = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))
        for _ in range(3):
            L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                            h=t.get("h"), W_down=t.get("W_down"), W_up=t.get("W_up"), out=bufs)
    torch.cuda.synchronize()
    del t, bufs
    torch.cuda.empty_cache()
    x = torch.empty(2 ** 28, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x).fill_(0.0)
    torch.cuda.synchronize()
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"profile_sample": workload, "copy_bytes": x.numel() * 4}))


def timed_steps(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def event_ring(n, torch):
    st = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    sp = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in st + sp:
        e.record()  # creates the HIP event handle
    torch.cuda.synchronize()
    return st, sp


def outer_median_us(fn, n, torch, flush, sink, graph):
    """Median µs of n calls of fn (graph: replays of fn captured in a HIP
    graph), each after a read of the flush buffer (cold cache), between two
    events on torch's stream recorded outside the call: the same clock for
    eager launches and graph replays."""
    fn()
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
    ev = event_ring(n, torch)
    for j in range(n):
        torch.sum(flush, dim=0, out=sink)
        ev[0][j].record()
        if g is not None:
            g.replay()
        else:
            fn()
        ev[1][j].record()
    torch.cuda.synchronize()
    tt = sorted(a.elapsed_time(b) for a, b in zip(*ev))
    del g
    return tt[len(tt) // 2] * 1e3


def copy_reference_gbs(n, torch, flush):
    """GB/s (bytes read + bytes written) of a plain device-to-device copy of
    the flush buffer into a second buffer of its size: what the runtime's own
    streaming copy reaches on this device, as context for the HBM
    fractions."""
    dst = torch.empty_like(flush)
    dst.copy_(flush)
    ev = event_ring(n, torch)
    for j in range(n):
        ev[0][j].record()
        dst.copy_(flush)
        ev[1][j].record()
    torch.cuda.synchronize()
    tt = sorted(a.elapsed_time(b) for a, b in zip(*ev))
    del dst
    return 2 * flush.numel() * flush.element_size() / (tt[len(tt) // 2] * 1e-3) / 1e9


def avg_ms(st, sp):
    return sum(a.elapsed_time(b) for a, b in zip(st, sp)) / len(st)


class Recorder:
    """Rings of (start, stop) events for some library steps: call j of the
    timed loop passes timing(j), so the library records ring slot j around
    that call's launches of each step (per call, no library state)."""

    def __init__(self, steps, n, torch):
        self.n = n
        self.rings = {sid: event_ring(n, torch) for sid in steps}
        self.j = 0

    def timing(self):
        j = self.j % self.n
        self.j += 1
        return {sid: (r[0][j], r[1][j]) for sid, r in self.rings.items()}

    def ms(self, sid):
        return avg_ms(*self.rings[sid])

    def times(self, sid):
        return [a.elapsed_time(b) for a, b in zip(*self.rings[sid])]


def _rate(flop, ms, peak):
    tf = flop / (ms * 1e-3) / 1e12
    return {"tflops": tf, "frac": tf / peak}


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------
STRATEGY_NAMES = {1: "union", 2: "compact", 3: "chunk_major"}
FUSED_KERNEL = {1: "k_attn_fwd", 2: "k_attn_fwd_sparse"}


def bench_prefill(name, steps, warmup, torch, L, strategy=0):
    """steps timed forwards of workload `name`: tokens/s, and per launch step
    its average device time (the library's events around that step in every
    timed call), algorithmic flops and MFMA fraction."""
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[name]
    t = make_inputs(wl, device="cuda")
    h, Wd, Wu = t.get("h"), t.get("W_down"), t.get("W_up")
    strat = L.fwd_strategy_of(L.make_problem(t["q"], t["k"], wl.S, wl.K, wl.W, h, Wd,
                                             strategy=strategy))
    cm = strat == L.FWD_CHUNK_MAJOR
    bufs = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, h, Wd, strategy=strat)
    rec = None

    def step():
        L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W, h=h,
                        W_down=Wd, W_up=Wu, out=bufs, strategy=strat,
                        timing=rec.timing() if rec else None)

    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    sids = ([L.STEP_QCAL] if wl.r else []) + [L.STEP_ROUTE, L.STEP_ATTN_FWD, L.STEP_PREP,
                                               L.STEP_WINDOW] + ([L.STEP_CHUNKS] if cm else [])
    rec = Recorder(sids, steps, torch)
    sec = timed_steps(step, steps, 0, torch)
    ms = {sid: rec.ms(sid) for sid in sids}
    rec = None
    peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    win_f, chk_f = fwd_algorithmic_flops(wl)
    kernels = {}
    if wl.r:
        kernels["qcal"] = {"kernel": "k_qcal", "ms": ms[L.STEP_QCAL],
                           "flop": qcal_algorithmic_flops(wl),
                           **_rate(qcal_algorithmic_flops(wl), ms[L.STEP_QCAL], peak)}
    rf = route_algorithmic_flops(wl)
    kernels["route"] = {"kernel": "k_route" + (" + k_route_scores" if wl.G > 1 else ""),
                        "ms": ms[L.STEP_ROUTE], "flop": rf, **_rate(rf, ms[L.STEP_ROUTE], peak)}
    kernels["prep"] = {"kernel": "k_vt_perm" + (" + inverse index + work items" if cm else ""),
                       "ms": ms[L.STEP_PREP]}
    if cm:
        kernels["chunks"] = {"kernel": "k_fwd_cm_chunks", "ms": ms[L.STEP_CHUNKS], "flop": chk_f,
                             **_rate(chk_f, ms[L.STEP_CHUNKS], peak)}
        kernels["window"] = {"kernel": "k_fwd_cm_window (window + fusion)",
                             "ms": ms[L.STEP_WINDOW], "flop": win_f,
                             **_rate(win_f, ms[L.STEP_WINDOW], peak)}
    else:
        kernels["window"] = {"kernel": FUSED_KERNEL[strat] + " (window + chunks + fusion)",
                             "ms": ms[L.STEP_WINDOW], "flop": win_f + chk_f,
                             **_rate(win_f + chk_f, ms[L.STEP_WINDOW], peak)}
    phases = {"together": {"ms": ms[L.STEP_ATTN_FWD], "flop": win_f + chk_f,
                           "launches": "every attention launch (V^T copy"
                                       + (", inverse index, chunks, window + fusion)" if cm
                                          else ", fused kernel)"),
                           **_rate(win_f + chk_f, ms[L.STEP_ATTN_FWD], peak)}}
    if cm:
        phases["chunks"] = dict(kernels["chunks"])
        phases["window"] = dict(kernels["window"])
    # the roofline of the longest single launch (the routing step of a GQA
    # problem is two launches and counts as one)
    dom = max((k for k in kernels if k != "prep"), key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    roof = {"bound": "mfma", "achieved": dk["tflops"], "peak": peak, "unit": "TFLOP/s",
            "frac": dk["frac"], "traffic": recorded_traffic(dom, wl.name), "kernel": dk["kernel"],
            "algorithmic_flop_per_launch": dk["flop"], "avg_launch_ms": dk["ms"]}
    out = {"workload": wl.name, "tokens_per_s": wl.B * wl.N / sec, "ms_per_step": sec * 1e3,
           "strategy": STRATEGY_NAMES[strat], "kernels": kernels, "phases": phases,
           "roofline": roof,
           "config": {"workload": wl.name, "batch": wl.B, "heads_q": wl.Hq, "heads_kv": wl.Hkv,
                      "head_dim": wl.d, "seq_len": wl.N, "chunk": wl.S, "top_k": wl.K,
                      "window": wl.W, "qcal_hidden": wl.D, "qcal_rank": wl.r,
                      "needle": wl.needle}}
    del t, bufs
    torch.cuda.empty_cache()
    return out, wl


def bench_decode(args, torch, L):
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[args.decode_workload]
    t = make_inputs(wl, device="cuda")
    bufs = L.decode_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))
    # a buffer larger than the 256 MiB last-level cache, read between steps so
    # that the step starts with none of its data cached (a read leaves clean
    # lines: no write-back of the flush competes with the step's reads)
    flush = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    rec = None

    def step():
        L.hils_decode(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                      seq_len=t["seq_len"], h=t.get("h"), W_down=t.get("W_down"),
                      W_up=t.get("W_up"), out=bufs, timing=rec.timing() if rec else None)

    for _ in range(max(1, args.warmup)):
        step()
    n = args.decode_steps
    rec = Recorder((L.STEP_DECODE,), n, torch)
    for _ in range(n):
        torch.sum(flush, dim=0, out=sink)
        step()
    torch.cuda.synchronize()
    times = sorted(rec.times(L.STEP_DECODE))
    rec = None
    med = times[len(times) // 2]
    nbytes = decode_bytes(wl)
    gbs = nbytes / (med * 1e-3) / 1e9
    out = {"workload": wl.name, "us_per_step": med * 1e3, "median_of": n, "cold_cache": True,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                        "traffic": recorded_traffic("decode", wl.name)}}

    def graph_median(fn):
        return outer_median_us(fn, n, torch, flush, sink, graph=True)

    out["graph_us_per_step"] = graph_median(step)
    # the eager step on the graph's clock (events outside the call), and a
    # plain 512 MiB device copy as the device's practical streaming rate
    out["eager_outer_us_per_step"] = outer_median_us(step, n, torch, flush, sink, graph=False)
    out["copy_reference"] = {"what": "device copy of a 512 MiB buffer (read + write bytes)",
                             "unit": "GB/s", "achieved": copy_reference_gbs(n, torch, flush)}
    if not args.no_paged:
        # the same caches as pages of one chunk each, in a shuffled order
        B, Hkv, N, d = t["k"].shape
        maxp = N // wl.S
        perm = torch.randperm(B * maxp, generator=torch.Generator().manual_seed(3)).reshape(B, maxp)
        perm = perm.to("cuda")
        pages = {}
        for name in ("k", "v"):
            pg = torch.empty((B * maxp, Hkv, wl.S, d), dtype=t[name].dtype, device="cuda")
            for b in range(B):
                pg[perm[b]] = t[name][b].reshape(Hkv, maxp, wl.S, d).permute(1, 0, 2, 3)
            pages[name] = pg
            del t[name]
        C = t["kL"].shape[2]
        kLp = torch.zeros((B * maxp, Hkv, d), dtype=t["kL"].dtype, device="cuda")
        ep = torch.zeros((B * maxp, Hkv), dtype=t["e"].dtype, device="cuda")
        kLp[perm[:, :C]] = t["kL"].permute(0, 2, 1, 3)
        ep[perm[:, :C]] = t["e"].permute(0, 2, 1)
        ptab = perm.to(torch.int32).contiguous()

        prec = None

        def pstep():
            L.hils_decode_paged(t["q"], pages["k"], pages["v"], ptab, t["seq_len"], kLp, ep, wl.S,
                                wl.K, wl.W, h=t.get("h"), W_down=t.get("W_down"),
                                W_up=t.get("W_up"), out=bufs,
                                timing=prec.timing() if prec else None)

        pstep()
        prec = Recorder((L.STEP_DECODE,), n, torch)
        for _ in range(n):
            torch.sum(flush, dim=0, out=sink)
            pstep()
        torch.cuda.synchronize()
        tt = sorted(prec.times(L.STEP_DECODE))
        prec = None
        out["paged_us_per_step"] = tt[len(tt) // 2] * 1e3
        out["paged_graph_us_per_step"] = graph_median(pstep)
        del pages, kLp, ep, ptab
    del t, bufs, flush, sink
    torch.cuda.empty_cache()
    return out


def bench_decode_long(args, torch, L):
    """The 4M-token decode (one sequence of 4194304 tokens, 16 heads, d = 64,
    K = 16, W = 512: 65528 distant landmarks per head): µs per step from a
    cold cache, eager and replayed from a HIP graph, against the HBM roofline
    of its 0.143 GB of algorithmic bytes."""
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["decode_4m"]
    t = make_inputs(wl, device="cuda")
    bufs = L.decode_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))
    flush = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    rec = None

    def step():
        L.hils_decode(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                      seq_len=t["seq_len"], h=t.get("h"), W_down=t.get("W_down"),
                      W_up=t.get("W_up"), out=bufs, timing=rec.timing() if rec else None)

    for _ in range(max(1, args.warmup)):
        step()
    n = args.decode_steps
    rec = Recorder((L.STEP_DECODE,), n, torch)
    for _ in range(n):
        torch.sum(flush, dim=0, out=sink)
        step()
    torch.cuda.synchronize()
    times = sorted(rec.times(L.STEP_DECODE))
    rec = None
    med = times[len(times) // 2]
    g_us = outer_median_us(step, n, torch, flush, sink, graph=True)
    e_us = outer_median_us(step, n, torch, flush, sink, graph=False)
    nbytes = decode_bytes(wl)
    gbs = nbytes / (med * 1e-3) / 1e9
    out = {"workload": wl.name, "us_per_step": med * 1e3, "graph_us_per_step": g_us,
           "eager_outer_us_per_step": e_us, "median_of": n, "cold_cache": True,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                        "traffic": recorded_traffic("decode", wl.name)}}
    del t, bufs, flush, sink
    torch.cuda.empty_cache()
    return out


def bench_train(args, torch, L):
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["train_345m"]
    t = make_inputs(wl, device="cuda")
    fb = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))
    gb = None
    rec = None

    def step():
        nonlocal gb
        tm = rec.timing() if rec else None
        o, lse, idx = L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                                      h=t["h"], W_down=t["W_down"], W_up=t["W_up"], out=fb,
                                      timing=tm)
        g = L.hils_attn_bwd(t["q"], t["k"], t["v"], t["kL"], t["e"], o, lse, idx, t["dO"], wl.S,
                            wl.K, wl.W, h=t["h"], W_down=t["W_down"], W_up=t["W_up"], out=gb,
                            timing=tm)
        if gb is None:
            gb = (g, L._workspace(L.make_problem(t["q"], t["k"], wl.S, wl.K, wl.W, t["h"],
                                                 t["W_down"]), L.OP_BWD, t["q"].device))

    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(3, args.steps // 2)
    rec = Recorder((L.STEP_ATTN_FWD, L.STEP_BWD), n, torch)
    sec = timed_steps(step, n, 0, torch)
    ms = {sid: rec.ms(sid) for sid in rec.rings}
    fl = train_algorithmic_flops(wl)
    tf = fl / sec / 1e12
    out = {"workload": wl.name, "tokens_per_s": wl.B * wl.N / sec, "ms_per_step": sec * 1e3,
           "attn_fwd_ms": ms[L.STEP_ATTN_FWD], "bwd_ms": ms[L.STEP_BWD],
           "mfma": {"achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tf / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flop_per_step": fl}}
    del t, fb, gb
    torch.cuda.empty_cache()
    return out


def bench_landmark(args, torch, L):
    """Landmark summary forward and backward at the 345M training shape."""
    from workloads import WORKLOADS, make_landmark_inputs
    wl = WORKLOADS["train_345m"]
    t = make_landmark_inputs(wl, device="cuda")
    dk = torch.zeros(t["k"].shape, dtype=torch.float32, device="cuda")
    # each call starts from a cache that holds none of its data and no dirty
    # lines (a read of a buffer larger than the last-level cache in between):
    # neither pays for the other's write-backs
    flush = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    rec = None

    def step():
        tm = rec.timing() if rec else None
        torch.sum(flush, dim=0, out=sink)
        L.hils_landmark_fwd(t["qL"], t["k"], wl.S, timing=tm)
        torch.sum(flush, dim=0, out=sink)
        L.hils_landmark_bwd(t["qL"], t["k"], t["dkL"], t["de"], wl.S, dk=dk, timing=tm)

    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(5, args.steps)
    rec = Recorder((L.STEP_LANDMARK_FWD, L.STEP_LANDMARK_BWD), n, torch)
    timed_steps(step, n, 0, torch)
    ms = {sid: rec.ms(sid) for sid in rec.rings}
    fb, bb = landmark_bytes(wl)
    fg = fb / (ms[L.STEP_LANDMARK_FWD] * 1e-3) / 1e9
    bgs = bb / (ms[L.STEP_LANDMARK_BWD] * 1e-3) / 1e9
    out = {"workload": wl.name + " landmark summary", "cold_cache": True,
           "fwd_us": ms[L.STEP_LANDMARK_FWD] * 1e3,
           "bwd_us": ms[L.STEP_LANDMARK_BWD] * 1e3,
           "hbm": {"fwd_gbs": fg, "bwd_gbs": bgs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac_fwd": fg / HBM_PEAK_GBS, "frac_bwd": bgs / HBM_PEAK_GBS,
                   "bytes_fwd": fb, "bytes_bwd": bb}}
    del t, dk, flush, sink
    torch.cuda.empty_cache()
    return out


def bench_hope(args, torch, L):
    """HoPE rotation of the 345M prefill query and key tensors (bf16
    [4, 16, 8192, 64] each, positions n, training length 8192), in place:
    an HBM stream that reads and writes every element once."""
    from workloads import WORKLOADS
    wl = WORKLOADS["prefill_345m"]
    g = torch.Generator(device="cuda").manual_seed(7)
    shape = (wl.B, wl.Hq, wl.N, wl.d)
    q = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)

    rec = None

    def step():
        L.hils_hope(q, None, train_len=wl.N, out=q, timing=rec.timing() if rec else None)
        L.hils_hope(k, None, train_len=wl.N, out=k, timing=rec.timing() if rec else None)

    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(5, args.steps)
    rec = Recorder((L.STEP_HOPE,), 2 * n, torch)
    timed_steps(step, n, 0, torch)
    ms = rec.ms(L.STEP_HOPE)
    nbytes = 2 * q.numel() * q.element_size()
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": wl.name + " HoPE rotation of q (and k)", "us_per_tensor": ms * 1e3,
           "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                   "bytes": nbytes}}
    del q, k
    torch.cuda.empty_cache()
    return out


def selection_locality(idx, wl, torch):
    """Chunk-id overlap of the selections (the paper's Fig. 7 measures): mean
    |T_i & T_i+1| / K of adjacent rows, and the mean union of the selections of
    M adjacent positions per KV head with the fraction of the visible distant
    chunks it is, for M = 16 and for the 128-position tile of the packed-union
    kernel."""
    a, b = idx[..., :-1, :], idx[..., 1:, :]
    full = (a >= 0).all(-1) & (b >= 0).all(-1)
    inter = torch.zeros(full.shape, dtype=torch.float32, device=idx.device)
    for j in range(idx.shape[-1]):
        inter += (a == b[..., j:j + 1]).sum(-1).float()
    out = {"adjacent_overlap": float(inter[full].mean()) / wl.K}
    B, Hkv, N, K = idx.shape
    for M in (16, 128 // wl.G):
        T = N // M
        x = idx[:, :, :T * M].reshape(B, Hkv, T, M * K)
        ok = (x >= 0).all(-1)
        xs, _ = torch.sort(x, -1)
        uniq = 1 + (xs[..., 1:] != xs[..., :-1]).sum(-1)
        last = torch.arange(T, device=idx.device) * M + M - 1
        nd = torch.clamp((last - wl.W + 1) // wl.S, min=1).to(torch.float32)
        out[f"union_m{M}"] = float(uniq[ok].float().mean())
        out[f"loaded_frac_m{M}"] = float((uniq.float() / nd)[ok].mean())
    return out



def bench_packing(args, torch, L):
    """The three forward strategies (packed union, compacted, chunk-major) on
    independent and on position-correlated queries (prefill_345m and
    prefill_345m_local): attention time of each, every launch included."""
    from workloads import WORKLOADS, make_inputs
    res = {}
    for name in ("prefill_345m", "prefill_345m_local"):
        wl = WORKLOADS[name]
        t = make_inputs(wl, device="cuda")
        r = None
        for sid in (L.FWD_UNION, L.FWD_COMPACT, L.FWD_CHUNK_MAJOR):
            fb = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"),
                               strategy=sid)
            rec = None

            def step():
                return L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                                       h=t["h"], W_down=t["W_down"], W_up=t["W_up"], out=fb,
                                       strategy=sid, timing=rec.timing() if rec else None)

            if r is None:
                r = selection_locality(step()[2], wl, torch)
            for _ in range(max(2, args.warmup)):
                step()
            torch.cuda.synchronize()
            n = max(5, args.steps)
            rec = Recorder((L.STEP_ATTN_FWD,), n, torch)
            timed_steps(step, n, 0, torch)
            r[f"attn_ms_{STRATEGY_NAMES[sid]}"] = rec.ms(L.STEP_ATTN_FWD)
            rec = None
            del fb
        res[name] = r
        del t
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_1p4b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-only", action="store_true",
                    help="run the oracle baselines only (no GPU needed) and print them")
    ap.add_argument("--cpu-positions", type=int, default=4096,
                    help="query positions per (batch, KV head) of the prefill oracle sample")
    ap.add_argument("--decode-workload", default="decode_7b_512k")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache decode timing")
    ap.add_argument("--legs",
                    default="prefill_345m,prefill_512k,decode,decode_long,train,landmark,hope,packing",
                    help="comma list of extra legs (the headline prefill always runs)")
    ap.add_argument("--profile-sample", action="store_true",
                    help="run the short fixed sample used for rocprofv3 counter passes and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)",
              file=sys.stderr)
        print(json.dumps({"error": "one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    legs = set(x for x in args.legs.split(",") if x)
    cpu = {}
    if not args.no_cpu_baseline and not args.profile_sample:
        cpu = cpu_baselines(args, legs)
    if args.cpu_only:
        print(json.dumps({"cpu_baseline": cpu}))
        return
    import torch
    import learnable_chunk_sparse_amd as L
    L.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.profile_sample:
        profile_sample(torch, L, args.workload)
        return
    head, wl = bench_prefill(args.workload, args.steps, args.warmup, torch, L)
    res = {}
    if "prefill_345m" in legs:
        r, _ = bench_prefill("prefill_345m", args.steps, args.warmup, torch, L)
        r2, _ = bench_prefill("prefill_345m", args.steps, args.warmup, torch, L,
                              strategy=L.FWD_CHUNK_MAJOR)
        r["chunk_major"] = {"ms_per_step": r2["ms_per_step"], "kernels": r2["kernels"],
                            "phases": r2["phases"]}
        res["prefill_345m"] = r
    if "prefill_512k" in legs:
        res["prefill_512k"], _ = bench_prefill("prefill_345m_512k", max(3, args.steps // 4),
                                               max(1, args.warmup), torch, L)
    if "decode" in legs:
        res["decode"] = bench_decode(args, torch, L)
        res["decode"]["cpu_baseline"] = cpu.get("decode")
        if "decode_long" in legs:
            res["decode"]["long_context"] = bench_decode_long(args, torch, L)
            res["decode"]["long_context"]["cpu_baseline"] = cpu.get("decode_long")
    if "train" in legs:
        res["train"] = bench_train(args, torch, L)
        res["train"]["cpu_baseline"] = cpu.get("train")
    if "landmark" in legs:
        res["landmark"] = bench_landmark(args, torch, L)
    if "hope" in legs:
        res["hope"] = bench_hope(args, torch, L)
    if "packing" in legs:
        res["packing"] = bench_packing(args, torch, L)
    line = {"metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
            "data": "synthetic (seeded counter-based generator)", "config": head["config"],
            "roofline": head["roofline"], "cpu_baseline": cpu.get("prefill"),
            "strategy": head["strategy"], "kernels": head["kernels"], "phases": head["phases"]}
    line.update(res)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
