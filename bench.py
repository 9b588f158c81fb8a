#!/usr/bin/env python3
"""Benchmark of the HiLS attention hot path on one MI355X.

Default workload: the 345M-shape prefill forward (batch 4, 16 heads, d 64,
8192 tokens, chunk 64, top-16, 512-token window, Q-Cal rank 32 from hidden
1024), bf16, seeded synthetic inputs resident in HBM. One step = one
hils_attn_fwd call: Q-Cal, routing (scores + GQA max + top-K), window and
selected-chunk attention, fusion.

Prints ONE JSON line: prefill tokens/s, the roofline of the dominant kernel
(its average duration measured with HIP events around each of its launches in
the timed region) and the fp64 CPU oracle timed on a bounded sample of the
same workload. Extra legs in the same line: "decode" (the 512K-context decode
step of 32 sequences, microseconds per step against the HBM roofline, cold
last-level cache; also replayed from a HIP graph and over a paged cache; and
the 4M-token single-sequence decode as "long_context"), "train" (forward + backward tokens/s) and "landmark" (the
landmark summary's forward and backward against the HBM roofline) and "packing"
(chunk-id overlap of adjacent queries and the two forward strategies on
independent and on position-correlated queries) and "hope" (the HoPE rotation
of the 345M prefill queries and keys against the HBM roofline).
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

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0


def n_distant(i, W, S):
    return max(0, (i - W + 1) // S)


def fwd_algorithmic_flops(wl):
    """Flops the method must do in the attention kernel: 4*d per
    (query head, attended token) over the window and the selected chunks."""
    win = 0
    chk = 0
    for i in range(wl.N):
        nd = n_distant(i, wl.W, wl.S)
        win += i + 1 - nd * wl.S
        chk += min(wl.K, nd) * wl.S
    per_pair = 4 * wl.d
    rows = wl.B * wl.Hq
    return rows * per_pair * win, rows * per_pair * chk


def route_algorithmic_flops(wl):
    tot = sum(n_distant(i, wl.W, wl.S) for i in range(wl.N))
    return wl.B * wl.Hq * 2 * wl.d * tot


def qcal_algorithmic_flops(wl):
    return wl.B * wl.N * wl.Hq * (2 * wl.r * wl.D + 2 * wl.d * wl.r) if wl.r else 0


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd__prefill_345m__hbm_traffic.md")
TRAFFIC_SOURCES = ["attn_fwd.hip", "attn_fwd_sparse.hip", "hils_common.h"]


def kernel_source_digest():
    """sha256 over the attention forward's source files (the counters in the
    traffic summary are only valid for the kernel they were taken on)."""
    import hashlib
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "learnable_chunk_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy
    calibration), or None when that summary is missing or was taken on
    different kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("- ") and ":" in line:
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("sources_sha256") != kernel_source_digest():
            return None
        return float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def profile_sample(torch, L, workload="prefill_345m"):
    """A short fixed run for rocprofv3 counter passes: three prefill forwards
    of the workload, then the calibration copy (1 GiB fp32 read, 1 GiB
    written) whose FETCH_SIZE / WRITE_SIZE scale the kernel's counters."""
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[workload]
    t = make_inputs(wl, device="cuda")
    bufs = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))
    for _ in range(3):
        L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W, h=t.get("h"),
                        W_down=t.get("W_down"), W_up=t.get("W_up"), out=bufs)
    torch.cuda.synchronize()
    del t, bufs
    x = torch.empty(2 ** 28, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x).fill_(0.0)
    torch.cuda.synchronize()
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"profile_sample": "done", "copy_bytes": x.numel() * 4}))


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


def cpu_baseline_prefill(wl, budget_s=12.0):
    """The fp64 oracle on stride-sampled query positions of a few (batch, KV
    group) pairs, run until about budget_s seconds of oracle time, then
    extrapolated to tokens/s of the whole workload (a token costs Hkv
    group-rows). The oracle is single-threaded NumPy/Python."""
    from workloads import make_group_inputs
    from oracle import hils_oracle as H
    stride = 64
    groups = [(b, (5 * b) % wl.Hkv) for b in range(wl.B)]
    rows_done = 0
    t_used = 0.0
    passes = 0
    for b, g in groups:
        t = make_group_inputs(wl, b, g)
        for offset in range(0, stride):
            rows = list(range(offset, wl.N, stride))
            t0 = time.perf_counter()
            H.hils_forward(t, wl.S, wl.K, wl.W, rows=rows)
            t_used += time.perf_counter() - t0
            rows_done += len(rows)
            passes += 1
            if t_used >= budget_s:
                break
        if t_used >= budget_s:
            break
    per_row = t_used / rows_done
    tok_s = 1.0 / (per_row * wl.Hkv)
    return {"value": tok_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows_done} query positions ({passes} passes of every {stride}th position "
                      f"over {min(len(groups), 1 + passes // 10)} (batch, KV head) pairs), "
                      f"{t_used:.1f} s of fp64 oracle time on one core, scaled by {wl.Hkv} KV "
                      f"heads per token"}


def bench_prefill(args, torch, L, W_):
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[args.workload]
    t = make_inputs(wl, device="cuda")
    bufs = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"))

    rec = None

    def step():
        L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W, h=t.get("h"),
                        W_down=t.get("W_down"), W_up=t.get("W_up"), out=bufs,
                        timing=rec.timing() if rec else None)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    rec = Recorder((L.STEP_QCAL, L.STEP_ROUTE, L.STEP_ATTN_FWD), args.steps, torch)
    sec = timed_steps(step, args.steps, 0, torch)
    k_ms = {sid: rec.ms(sid) for sid in rec.rings}
    win_f, chk_f = fwd_algorithmic_flops(wl)
    attn_flops = win_f + chk_f
    attn_tf = attn_flops / (k_ms[L.STEP_ATTN_FWD] * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    tokens = wl.B * wl.N
    res = {
        "metric": "HiLS prefill tokens/s (345M-shape forward: Q-Cal + routing + window/chunk "
                  "attention + fusion)",
        "value": tokens / sec, "unit": "tokens/s", "ms_per_step": sec * 1e3,
        "roofline": {"bound": "mfma", "achieved": attn_tf, "peak": peak, "unit": "TFLOP/s",
                     "frac": attn_tf / peak, "traffic": recorded_traffic(),
                     "kernel": "k_attn_fwd (window + selected chunks + fusion)",
                     "algorithmic_flop_per_launch": attn_flops,
                     "avg_launch_ms": k_ms[L.STEP_ATTN_FWD]},
        "steps_ms": {"qcal": k_ms[L.STEP_QCAL], "route": k_ms[L.STEP_ROUTE],
                     "attn_fwd": k_ms[L.STEP_ATTN_FWD]},
        "step_tflops": {
            "qcal": qcal_algorithmic_flops(wl) / (k_ms[L.STEP_QCAL] * 1e-3) / 1e12,
            "route": route_algorithmic_flops(wl) / (k_ms[L.STEP_ROUTE] * 1e-3) / 1e12,
            "attn_window_plus_chunks": attn_tf},
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "config": {"workload": wl.name, "batch": wl.B, "heads_q": wl.Hq, "heads_kv": wl.Hkv,
                   "head_dim": wl.d, "seq_len": wl.N, "chunk": wl.S, "top_k": wl.K,
                   "window": wl.W, "qcal_hidden": wl.D, "qcal_rank": wl.r},
    }
    del t, bufs
    torch.cuda.empty_cache()
    return res, wl


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
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes}}

    def graph_median(fn):
        """Median µs of replays of fn captured in a HIP graph (cold cache)."""
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        ev = event_ring(n, torch)
        for j in range(n):
            torch.sum(flush, dim=0, out=sink)
            ev[0][j].record()
            g.replay()
            ev[1][j].record()
        torch.cuda.synchronize()
        tt = sorted(a.elapsed_time(b) for a, b in zip(*ev))
        del g
        return tt[len(tt) // 2] * 1e3

    out["graph_us_per_step"] = graph_median(step)
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
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    ev = event_ring(n, torch)
    for j in range(n):
        torch.sum(flush, dim=0, out=sink)
        ev[0][j].record()
        g.replay()
        ev[1][j].record()
    torch.cuda.synchronize()
    tg = sorted(a.elapsed_time(b) for a, b in zip(*ev))
    nbytes = decode_bytes(wl)
    gbs = nbytes / (med * 1e-3) / 1e9
    out = {"workload": wl.name, "us_per_step": med * 1e3, "graph_us_per_step": tg[len(tg) // 2] * 1e3,
           "median_of": n, "cold_cache": True,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes}}
    del g, t, bufs, flush, sink
    torch.cuda.empty_cache()
    return out


def train_algorithmic_flops(wl):
    """Forward 4*d and backward 10*d flops per (query head, attended token)
    (backward: S, dP, dq, dk and dv products), plus the routing scores."""
    win_f, chk_f = fwd_algorithmic_flops(wl)
    attn = win_f + chk_f
    return attn + attn * 10 // 4 + route_algorithmic_flops(wl)


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
    """The two forward strategies (packed union, compacted) on independent and
    on position-correlated queries (prefill_345m and prefill_345m_local)."""
    from workloads import WORKLOADS, make_inputs
    res = {}
    for name in ("prefill_345m", "prefill_345m_local"):
        wl = WORKLOADS[name]
        t = make_inputs(wl, device="cuda")
        rec = None
        strat = L.FWD_AUTO

        def step():
            fb = L.fwd_buffers(t["q"], t["k"], wl.S, wl.K, wl.W, t.get("h"), t.get("W_down"),
                               strategy=strat) if bufs.get(strat) is None else bufs[strat]
            bufs[strat] = fb
            return L.hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W,
                                   h=t["h"], W_down=t["W_down"], W_up=t["W_up"], out=fb,
                                   strategy=strat, timing=rec.timing() if rec else None)

        bufs = {}
        r = selection_locality(step()[2], wl, torch)
        for sname, sid in (("union", L.FWD_UNION), ("compact", L.FWD_COMPACT)):
            strat = sid
            rec = None
            for _ in range(max(2, args.warmup)):
                step()
            torch.cuda.synchronize()
            n = max(5, args.steps)
            rec = Recorder((L.STEP_ATTN_FWD,), n, torch)
            timed_steps(step, n, 0, torch)
            r[f"attn_ms_{sname}"] = rec.ms(L.STEP_ATTN_FWD)
            rec = None
            bufs.pop(sid, None)
        res[name] = r
        del t, bufs
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_345m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-decode", action="store_true", help="skip the 512K decode leg")
    ap.add_argument("--decode-workload", default="decode_7b_512k")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache decode timing")
    ap.add_argument("--no-train", action="store_true", help="skip the training (fwd+bwd) leg")
    ap.add_argument("--legs", default="prefill,decode,decode_long,train,landmark,packing,hope",
                    help="comma list of legs to run (prefill is always reported)")
    ap.add_argument("--profile-sample", action="store_true",
                    help="run the short fixed sample used for rocprofv3 counter passes and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import learnable_chunk_sparse_amd as L
    L.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.profile_sample:
        profile_sample(torch, L, args.workload)
        return
    res, wl = bench_prefill(args, torch, L, None)
    legs = set(args.legs.split(","))
    if not args.no_decode and "decode" in legs:
        res["decode"] = bench_decode(args, torch, L)
        if "decode_long" in legs:
            res["decode"]["long_context"] = bench_decode_long(args, torch, L)
    if not args.no_train and "train" in legs:
        res["train"] = bench_train(args, torch, L)
    if "landmark" in legs:
        res["landmark"] = bench_landmark(args, torch, L)
    if "hope" in legs:
        res["hope"] = bench_hope(args, torch, L)
    if "packing" in legs:
        res["packing"] = bench_packing(args, torch, L)
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_prefill(wl, args.cpu_budget)
    res["vs_baseline"] = None
    line = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": res.pop("vs_baseline"), "dtype": res.pop("dtype"),
            "data": "synthetic (seeded counter-based generator)", "config": res.pop("config")}
    line.update(res)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
