"""Shared helpers for the parity tests (GPU library vs the fp64 oracle)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import hils_oracle as H

# tolerances stated for the method: bf16 inputs with fp32 accumulation, fp32 inputs
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3), "fp32": dict(max_abs=1e-5, mean_abs=1e-5)}
LSE_TOL = {"bf16": 2e-3, "fp32": 1e-5}
NEAR_TIE_REL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_dev(t: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}


def check_topk_row(gpu_set, sel_sorted, order, K, nd):
    """Admissibility of one row's GPU selection against the oracle's ranking.

    Exact agreement unless the oracle's K-th and (K+1)-th scores differ by
    less than 1e-4 relative (floor 1); then the GPU set must contain every
    chunk scoring above the tied band and only chunks inside or above it.
    Returns (ok, near_tie)."""
    gpu = sorted(int(c) for c in gpu_set if c >= 0)
    keff = min(K, nd)
    if len(gpu) != keff:
        return False, False
    if keff == nd:
        return gpu == list(range(nd)), False
    sK, sK1 = sel_sorted[keff - 1], sel_sorted[keff]
    band = NEAR_TIE_REL * max(abs(sK), abs(sK1), 1.0)
    ref = sorted(int(c) for c in order[:keff])
    if sK - sK1 >= band:
        return gpu == ref, False
    score = {int(c): s for c, s in zip(order, sel_sorted)}
    above = {int(c) for c, s in zip(order, sel_sorted) if s > sK + band}
    okset = all(c in score and score[c] >= sK - band for c in gpu) and above <= set(gpu)
    return okset, True


def grad_tol(dtype, ref):
    """The bar for a gradient. bf16: the method's absolute bar (max-abs 2e-2,
    mean-abs 2e-3). fp32: 1e-5, absolute where |ref| <= 1 and relative to
    |ref| above (checked element by element). The backward sums its fp32
    terms in one fixed order (the inverse index is a stable sort and the
    chunk terms of a row are added in a fixed sequence), and the rounding of
    an fp32 sum grows with its magnitude: n terms of a sum S carry up to about
    n u |S| (u = 2^-24); 1e-5 relative is ~170 ulps, the bound for a few
    hundred terms such as dv's key rows."""
    t = dict(TOL[dtype])
    if dtype == "fp32":
        t["rel_floor"] = 1.0
    return t


def compare(name, got, ref, dtype, tol=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    t = tol or TOL[dtype]
    if "rel_floor" in t:
        # element by element: absolute up to |ref| = rel_floor, relative above
        err = err / np.maximum(t["rel_floor"], np.abs(ref))
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} (tol {t['max_abs']:.0e}/{t['mean_abs']:.0e})")
    assert mx <= t["max_abs"], f"{name}: max abs err {mx} > {t['max_abs']}"
    assert mean <= t["mean_abs"], f"{name}: mean abs err {mean} > {t['mean_abs']}"
    return mx, mean


def fwd_parity(t_cpu: dict, gpu_out, S, K, W, dtype, rows=None, batches=None, groups=None,
               label=""):
    """Check o / lse / topk_idx of a GPU forward against the oracle on the
    chosen rows: selections first (exact or admissible near-tie), then the
    outputs against the oracle rerun on the GPU's (admissible) selection."""
    o, lse, idx = (x.detach().cpu() for x in gpu_out)
    idx = idx.numpy()
    B, Hq, N, d = t_cpu["q"].shape
    Hkv = t_cpu["k"].shape[1]
    G = Hq // Hkv
    rows = list(range(N)) if rows is None else list(rows)
    batches = list(range(B)) if batches is None else list(batches)
    groups = list(range(Hkv)) if groups is None else list(groups)
    rt = H.hils_route(t_cpu, S, K, W, rows=rows, batches=batches, groups=groups)
    nt = 0
    for b in batches:
        for g in groups:
            for i in rows:
                sel_sorted, order = rt["ranked"][(b, g, i)]
                ok, tie = check_topk_row(idx[b, g, i], sel_sorted, order, K, H.n_distant(i, W, S))
                nt += tie
                assert ok, (f"{label} topk mismatch at b={b} g={g} i={i}: gpu={idx[b, g, i].tolist()} "
                            f"oracle={rt['topk'][b, g, i].tolist()}")
    say(f"{label}: topk sets ok on {len(batches) * len(groups) * len(rows)} rows ({nt} near-ties)")
    ref = H.hils_forward(t_cpu, S, K, W, rows=rows, batches=batches, groups=groups, forced_topk=idx)
    sel_o = []
    sel_r = []
    sel_l = []
    sel_lr = []
    for b in batches:
        for g in groups:
            hs = slice(g * G, (g + 1) * G)
            sel_o.append(o[b, hs][:, rows].to(torch.float64).numpy())
            sel_r.append(ref["o"][b, hs][:, rows])
            sel_l.append(lse[b, hs][:, rows].to(torch.float64).numpy())
            sel_lr.append(ref["lse"][b, hs][:, rows])
    compare(f"{label} o", np.stack(sel_o), np.stack(sel_r), dtype)
    lt = LSE_TOL[dtype]
    compare(f"{label} lse", np.stack(sel_l), np.stack(sel_lr), dtype, dict(max_abs=lt, mean_abs=lt))
