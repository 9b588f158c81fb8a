"""Seeded synthetic inputs for the HiLS attention hot path.

This module only draws numbers and lays them out. It holds none of the
method's arithmetic, so both the CPU oracle and the GPU path can take their
inputs from it without sharing any of the computation being checked.

Every tensor is cut into slabs (one per batch element and head, or per head
for weights). Each element of a slab is a pure function of
(seed, tensor id, batch index, head index, element counter): a counter-based
generator built on the "lowbias32" integer hash (C. Wellons, "Prospecting for
hash functions", 2018), evaluated with exact integer arithmetic in torch.
Floating-point values are formed with exact fp32 operations plus a single
correctly rounded multiply, so the same call on the CPU or on a GPU yields
bit-identical tensors, and any slab (or any row of one) can be regenerated on
its own, which is how the oracle re-creates the few slabs it checks at
full-size shapes.

Distributions:
  * "normal": N(0,1) by inversion. The top 22 bits of the hash pick one of
    2^22 equal-probability bins, and the value is the N(0,1) quantile at the
    bin's midpoint probability (k + 1/2) / 2^22: a table computed once in
    fp64 (scipy's inverse normal CDF) and rounded to fp32. Every bin has the
    probability of the normal law, so the tails are the normal tails down to
    probability 2^-23 (|z| up to 5.17).
  * "uniform(a)": U(-a, a) with a a power of two, on a 2^-22*a grid (exact).
Values are drawn in fp32 and rounded to bf16 (round to nearest even) for the
bf16 workloads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence

import torch

M32 = 0xFFFFFFFF

# tensor ids used in the slab keys
TID = dict(q=0, k=1, v=2, kL=3, e=4, h=5, W_down=6, W_up=7, dO=8, needle=9, qL=10, dkL=11, de=12)


# --------------------------------------------------------------------------
# counter-based generator
# --------------------------------------------------------------------------
def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32).

    Split into 16-bit halves so that no intermediate overflows int64."""
    lo = x & 0xFFFF
    hi = x >> 16
    return ((lo * c) + (((hi * c) & 0xFFFF) << 16)) & M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def slab_key(seed: int, tensor: str, b: int, head: int) -> int:
    k = _mix32_int(seed * 0x9E3779B1 + 0x1234567)
    k = _mix32_int(k ^ (TID[tensor] * 0x85EBCA6B + 0x2F))
    k = _mix32_int(k ^ (b * 0xC2B2AE35 + 0x51))
    k = _mix32_int(k ^ (head * 0x27D4EB2F + 0x77))
    return k


def _hash(counter: torch.Tensor, key: int, stream: int) -> torch.Tensor:
    x = (counter * 2 + stream) & M32
    x = _mix32(x ^ key)
    x = _mix32(x ^ ((key * 0x9E3779B1 + 0x632BE5AB) & M32))
    return x


NORMAL_BITS = 22
_NORMAL_TABLES: Dict[str, torch.Tensor] = {}


def normal_table(device="cpu") -> torch.Tensor:
    """fp32 N(0,1) quantiles at the probabilities (k + 1/2) / 2^22,
    k = 0 .. 2^22 - 1 (computed in fp64, rounded once), cached per device."""
    key = str(torch.device(device))
    if key not in _NORMAL_TABLES:
        if "cpu" not in _NORMAL_TABLES:
            import numpy as np
            from scipy.special import ndtri
            n = 1 << NORMAL_BITS
            p = (np.arange(n, dtype=np.float64) + 0.5) / n
            _NORMAL_TABLES["cpu"] = torch.from_numpy(ndtri(p).astype(np.float32))
        _NORMAL_TABLES[key] = _NORMAL_TABLES["cpu"].to(device)
    return _NORMAL_TABLES[key]


def normal_at(key: int, counter: torch.Tensor) -> torch.Tensor:
    """N(0,1) in fp32 at the given int64 counters (inversion through the
    quantile table: the same value on any device)."""
    h = _hash(counter, key, 0) >> (32 - NORMAL_BITS)
    return normal_table(counter.device)[h]


def uniform_at(key: int, counter: torch.Tensor, a: float) -> torch.Tensor:
    """U(-a, a) in fp32 (a a power of two) at the given counters, exact."""
    assert a > 0 and math.log2(a) == int(math.log2(a))
    v = _hash(counter, key, 0) >> 9  # 23 bits
    x = (2 * v + 1).to(torch.float32)  # exact (< 2^24)
    return x * (a * 2.0 ** -23) - a


def _counters(n: int, device, start: int = 0) -> torch.Tensor:
    return torch.arange(start, start + n, dtype=torch.int64, device=device)


# --------------------------------------------------------------------------
# workload descriptions (sizes and distributions only)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str  # "fp32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int  # tokens (prefill) or cache capacity (decode)
    S: int
    K: int
    W: int
    D: int = 0
    r: int = 0
    e_range: float = 1.0
    w_std: float = 0.02
    mode: str = "prefill"  # "prefill" | "decode" | "train"
    needle: str = "none"  # "none" | "chunk7" | "segments" | "decode_random"
    seq_len: Optional[Sequence[int]] = None  # decode: per-sequence lengths (default N)
    e_shift: float = 0.0  # added to every entropy bias (chunk-path-dominant variants)
    q_corr: float = 0.0  # AR(1) correlation of consecutive query positions (0: independent)
    notes: str = ""

    @property
    def C(self) -> int:
        return self.N // self.S

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, shaped like the paper's 345M / 1.4B / 7B settings
# (Fig. 6 of the paper: chunk 64, 512-token window; top-k values per workload).
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", seed=0, dtype="fp32", B=1, Hq=1, Hkv=1, d=64, N=2048, S=64,
                     K=4, W=128, e_range=1.0, needle="chunk7"),
    "prefill_345m": Workload("prefill_345m", seed=1, dtype="bf16", B=4, Hq=16, Hkv=16, d=64,
                             N=8192, S=64, K=16, W=512, D=1024, r=32, e_range=2.0),
    "prefill_1p4b": Workload("prefill_1p4b", seed=2, dtype="bf16", B=1, Hq=32, Hkv=8, d=128,
                             N=131072, S=64, K=16, W=1024, D=2048, r=32, e_range=2.0,
                             needle="segments"),
    "decode_7b_512k": Workload("decode_7b_512k", seed=3, dtype="bf16", B=32, Hq=32, Hkv=8,
                               d=128, N=524288, S=64, K=32, W=1024, e_range=2.0,
                               mode="decode"),
    "decode_4m": Workload("decode_4m", seed=3, dtype="bf16", B=1, Hq=16, Hkv=16, d=64,
                          N=4194304, S=64, K=16, W=512, e_range=2.0, mode="decode",
                          needle="decode_random"),
    "train_345m": Workload("train_345m", seed=4, dtype="bf16", B=8, Hq=16, Hkv=16, d=64,
                           N=8192, S=64, K=16, W=512, D=1024, r=32, e_range=2.0,
                           mode="train"),
    # the paper's long-context prefill measurement (Fig. 6): the 345M shape at
    # batch 1, chunk 64, top-32, a 512-token window, 524288 tokens; one
    # planted needle chunk per 16384-token segment
    "prefill_345m_512k": Workload("prefill_345m_512k", seed=5, dtype="bf16", B=1, Hq=16, Hkv=16,
                                  d=64, N=524288, S=64, K=32, W=512, D=1024, r=32, e_range=2.0,
                                  needle="segments"),
    # the 345M prefill with queries correlated along positions (AR(1), 0.97): adjacent
    # queries share ~92 % of their top-16, the locality the paper measures on trained
    # models (Fig. 7) and that independent queries lack
    "prefill_345m_local": Workload("prefill_345m_local", seed=1, dtype="bf16", B=4, Hq=16,
                                   Hkv=16, d=64, N=8192, S=64, K=16, W=512, D=1024, r=32,
                                   e_range=2.0, q_corr=0.97),
}


# --------------------------------------------------------------------------
# slab generation
# --------------------------------------------------------------------------
def _round(x: torch.Tensor, wl: Workload) -> torch.Tensor:
    return x.to(wl.torch_dtype)


def gen_slab(wl: Workload, tensor: str, b: int, head: int, shape, device="cpu",
             rows: Optional[torch.Tensor] = None, row_len: Optional[int] = None) -> torch.Tensor:
    """One slab of a raw (needle-free) input, in the workload's dtype.

    `rows` selects rows of a 2-D slab (row length `row_len`) without
    generating the rest."""
    key = slab_key(wl.seed, tensor, b, head)
    if rows is None:
        n = 1
        for s in shape:
            n *= s
        ctr = _counters(n, device)
    else:
        rows = rows.to(device=device, dtype=torch.int64)
        ctr = (rows[:, None] * row_len + torch.arange(row_len, device=device)[None, :]).reshape(-1)
        shape = (rows.numel(), row_len)
    if tensor == "e":
        x = uniform_at(key, ctr, wl.e_range)
        if wl.e_shift:
            x = x + wl.e_shift
    elif tensor in ("W_down", "W_up"):
        x = normal_at(key, ctr) * torch.tensor(wl.w_std, dtype=torch.float32, device=device)
    else:
        x = normal_at(key, ctr)
    return _round(x.reshape(shape), wl)


def correlate_positions(z: torch.Tensor, rho: float) -> torch.Tensor:
    """AR(1) filter along the position axis (dim -2) in fp32, unit variance
    kept: x_0 = z_0, x_i = rho x_{i-1} + sqrt(1 - rho^2) z_i. Plain fp32
    multiplies and adds in a fixed order, so CPU and GPU agree bit for bit."""
    a = torch.tensor(math.sqrt(1.0 - rho * rho), dtype=torch.float32, device=z.device)
    r = torch.tensor(rho, dtype=torch.float32, device=z.device)
    x = torch.empty_like(z)
    x[..., 0, :] = z[..., 0, :]
    for i in range(1, z.shape[-2]):
        x[..., i, :] = torch.add(torch.mul(x[..., i - 1, :], r), torch.mul(z[..., i, :], a))
    return x


def correlated_queries(wl: Workload, slabs, device="cpu") -> torch.Tensor:
    """Query slabs [(b, h), ...] -> [len, N, d] of a workload with q_corr > 0:
    each slab's normal draw filtered along positions (elementwise identical
    whether slabs are filtered together or alone), then rounded."""
    N, d = wl.N, wl.d
    z = torch.empty((len(slabs), N, d), dtype=torch.float32, device=device)
    for j, (b, h) in enumerate(slabs):
        z[j] = normal_at(slab_key(wl.seed, "q", b, h), _counters(N * d, device)).reshape(N, d)
    return _round(correlate_positions(z, wl.q_corr), wl)


def _alloc(shape, wl, device):
    return torch.empty(shape, dtype=wl.torch_dtype, device=device)


def needle_chunk_decode(wl: Workload, b: int, head: int) -> int:
    """The planted chunk of a decode sequence: uniform over its distant chunks."""
    n = seq_lens(wl)[b]
    nd = max(0, (n - 1 - wl.W + 1) // wl.S)
    return _mix32_int(slab_key(wl.seed, "needle", b, head)) % max(nd, 1)


def needle_chunks_segments(wl: Workload, g: int):
    """Planted chunks of the long prefill: one per 16384-token segment."""
    seg = 16384
    per = seg // wl.S
    out = []
    for s in range(wl.N // seg):
        out.append(s * per + _mix32_int(slab_key(wl.seed, "needle", s, g)) % per)
    return out


def seq_lens(wl: Workload):
    if wl.seq_len is not None:
        return list(wl.seq_len)
    return [wl.N] * wl.B


def make_inputs(wl: Workload, device="cpu", with_grad_inputs: Optional[bool] = None) -> dict:
    """All inputs of a workload as contiguous tensors on `device`.

    Layouts: q [B,Hq,N,d] (decode: [B,Hq,d]), k/v [B,Hkv,N,d], kL [B,Hkv,C,d],
    e [B,Hkv,C], h [B,N,D] (decode: [B,D]), W_down [Hq,r,D], W_up [Hq,d,r],
    dO [B,Hq,N,d]. Prefill needles are planted after the raw draw."""
    B, Hq, Hkv, d, N, C = wl.B, wl.Hq, wl.Hkv, wl.d, wl.N, wl.C
    out = {}
    dec = wl.mode == "decode"
    q = _alloc((B, Hq, d) if dec else (B, Hq, N, d), wl, device)
    k = _alloc((B, Hkv, N, d), wl, device)
    v = _alloc((B, Hkv, N, d), wl, device)
    kL = _alloc((B, Hkv, C, d), wl, device)
    e = _alloc((B, Hkv, C), wl, device)
    if wl.q_corr > 0 and not dec:
        q.copy_(correlated_queries(wl, [(b, h) for b in range(B) for h in range(Hq)],
                                   device).reshape(B, Hq, N, d))
    for b in range(B):
        for h in range(Hq):
            if not (wl.q_corr > 0 and not dec):
                q[b, h] = gen_slab(wl, "q", b, h, q.shape[2:], device)
        for g in range(Hkv):
            k[b, g] = gen_slab(wl, "k", b, g, (N, d), device)
            v[b, g] = gen_slab(wl, "v", b, g, (N, d), device)
            kL[b, g] = gen_slab(wl, "kL", b, g, (C, d), device)
            e[b, g] = gen_slab(wl, "e", b, g, (C,), device)
    out.update(q=q, k=k, v=v, kL=kL, e=e)
    if wl.r > 0:
        hs = _alloc((B, wl.D) if dec else (B, N, wl.D), wl, device)
        for b in range(B):
            hs[b] = gen_slab(wl, "h", b, 0, hs.shape[1:], device)
        Wd = _alloc((Hq, wl.r, wl.D), wl, device)
        Wu = _alloc((Hq, d, wl.r), wl, device)
        for h in range(Hq):
            Wd[h] = gen_slab(wl, "W_down", 0, h, (wl.r, wl.D), device)
            Wu[h] = gen_slab(wl, "W_up", 0, h, (d, wl.r), device)
        out.update(h=hs, W_down=Wd, W_up=Wu)
    if with_grad_inputs or (with_grad_inputs is None and wl.mode == "train"):
        dO = _alloc((B, Hq, N, d), wl, device)
        for b in range(B):
            for h in range(Hq):
                dO[b, h] = gen_slab(wl, "dO", b, h, (N, d), device)
        out["dO"] = dO
    plant_needles(wl, out)
    if dec:
        out["seq_len"] = torch.tensor(seq_lens(wl), dtype=torch.int32, device=device)
    return out


def make_landmark_inputs(wl: Workload, device="cpu", keys: bool = True) -> dict:
    """Inputs of the landmark summary for a workload: the keys k
    [B,Hkv,N,d] (the same slabs as make_inputs, without needles; omitted when
    keys=False), one landmark query per complete chunk and KV head qL
    [B,Hkv,C,d] (normal, workload dtype), and upstream gradients dkL
    [B,Hkv,C,d] and de [B,Hkv,C] (normal, fp32)."""
    B, Hkv, d, N, C = wl.B, wl.Hkv, wl.d, wl.N, wl.C
    qL = _alloc((B, Hkv, C, d), wl, device)
    dkL = torch.empty((B, Hkv, C, d), dtype=torch.float32, device=device)
    de = torch.empty((B, Hkv, C), dtype=torch.float32, device=device)
    k = _alloc((B, Hkv, N, d), wl, device) if keys else None
    for b in range(B):
        for g in range(Hkv):
            qL[b, g] = gen_slab(wl, "qL", b, g, (C, d), device)
            dkL[b, g] = normal_at(slab_key(wl.seed, "dkL", b, g), _counters(C * d, device)).reshape(C, d)
            de[b, g] = normal_at(slab_key(wl.seed, "de", b, g), _counters(C, device))
            if keys:
                k[b, g] = gen_slab(wl, "k", b, g, (N, d), device)
    out = dict(qL=qL, dkL=dkL, de=de)
    if keys:
        out["k"] = k
    return out


def _unit(x64: torch.Tensor) -> torch.Tensor:
    return x64 / torch.linalg.vector_norm(x64)


def plant_needles(wl: Workload, t: dict) -> None:
    """Plant the workload's needle chunks into the generated tensors (in place).

    A needle chunk has all of its keys equal to 3*sqrt(d)*u for a unit vector u
    pointing along a query, and its landmark key along that same query, so the
    chunk should be selected by (and dominate for) that query."""
    if wl.needle == "none":
        return
    for b in range(t["q"].shape[0]):
        for g in range(t["k"].shape[1]):
            _plant_group(wl, t, b, g, b, g)


def _plant_group(wl: Workload, t: dict, tb: int, tg: int, b: int, g: int) -> None:
    """Plant the needles of (batch b, KV group g) of the workload into slot
    (tb, tg) of the tensors in t (whose q holds that group's heads at
    tg*G .. tg*G+G-1)."""
    d, S, G = wl.d, wl.S, wl.G
    rd = math.sqrt(d)
    dec = wl.mode == "decode"
    if wl.needle == "chunk7":
        ql = t["q"][tb, tg * G, wl.N - 1].to(torch.float64).cpu()
        key = (3.0 * rd * _unit(ql)).to(wl.torch_dtype)
        t["k"][tb, tg, 7 * S:8 * S] = key.to(t["k"].device)[None, :]
        t["kL"][tb, tg, 7] = ql.to(wl.torch_dtype).to(t["kL"].device)
    elif wl.needle == "segments":
        seg = 16384
        for s, c in enumerate(needle_chunks_segments(wl, g)):
            acc = torch.zeros(d, dtype=torch.float64)
            for hh in range(G):
                acc += t["q"][tb, tg * G + hh, s * seg:(s + 1) * seg].to(torch.float64).cpu().sum(dim=0)
            u = _unit(acc)
            t["k"][tb, tg, c * S:(c + 1) * S] = (3.0 * rd * u).to(wl.torch_dtype).to(t["k"].device)[None, :]
            t["kL"][tb, tg, c] = (rd * u).to(wl.torch_dtype).to(t["kL"].device)
    elif wl.needle == "decode_random":
        c = needle_chunk_decode(wl, b, g)
        ql = (t["q"][tb, tg * G] if dec else t["q"][tb, tg * G, -1]).to(torch.float64).cpu()
        t["k"][tb, tg, c * S:(c + 1) * S] = (3.0 * rd * _unit(ql)).to(wl.torch_dtype).to(t["k"].device)[None, :]
        t["kL"][tb, tg, c] = ql.to(wl.torch_dtype).to(t["kL"].device)
    else:
        raise ValueError(wl.needle)


def make_group_inputs(wl: Workload, b: int, g: int, h_rows: Optional[Sequence[int]] = None,
                      kv_len: Optional[int] = None, kv_rows: Optional[Sequence[int]] = None) -> dict:
    """The slabs of one (batch b, KV group g) as a stand-alone CPU problem
    (B = 1, Hkv = 1, Hq = G), bit-identical to the same slabs of
    make_inputs(wl) on any device. HiLS rows of one group depend on nothing
    else, so the oracle can check a full-size run group by group.

    h_rows: generate only these rows of the hidden state (others are NaN).
    kv_len: decode only, generate only the first kv_len cache tokens.
    kv_rows: generate only these key/value rows (others are NaN); needle
    rows are always planted."""
    G, d, N, C = wl.G, wl.d, wl.N, wl.C
    dec = wl.mode == "decode"
    n = N if kv_len is None else kv_len
    out = {}
    if wl.q_corr > 0 and not dec:
        out["q"] = correlated_queries(wl, [(b, g * G + hh) for hh in range(G)])[None]
    else:
        qs = [gen_slab(wl, "q", b, g * G + hh, (d,) if dec else (N, d)) for hh in range(G)]
        out["q"] = torch.stack(qs)[None]
    if kv_rows is None:
        out["k"] = gen_slab(wl, "k", b, g, (n, d), rows=torch.arange(n), row_len=d)[None, None]
        out["v"] = gen_slab(wl, "v", b, g, (n, d), rows=torch.arange(n), row_len=d)[None, None]
    else:
        rr = torch.tensor(sorted(set(int(i) for i in kv_rows)), dtype=torch.int64)
        for name in ("k", "v"):
            full = torch.full((n, d), float("nan"), dtype=wl.torch_dtype)
            if rr.numel():
                full[rr] = gen_slab(wl, name, b, g, None, rows=rr, row_len=d)
            out[name] = full[None, None]
    out["kL"] = gen_slab(wl, "kL", b, g, (C, d))[None, None]
    out["e"] = gen_slab(wl, "e", b, g, (C,))[None, None]
    if wl.r > 0:
        if dec:
            out["h"] = gen_slab(wl, "h", b, 0, (wl.D,))[None]
        elif h_rows is None:
            out["h"] = gen_slab(wl, "h", b, 0, (N, wl.D))[None]
        else:
            hr = torch.full((N, wl.D), float("nan"), dtype=wl.torch_dtype)
            rows = torch.tensor(sorted(set(int(i) for i in h_rows)), dtype=torch.int64)
            hr[rows] = gen_slab(wl, "h", b, 0, None, rows=rows, row_len=wl.D)
            out["h"] = hr[None]
        out["W_down"] = torch.stack([gen_slab(wl, "W_down", 0, g * G + hh, (wl.r, wl.D)) for hh in range(G)])
        out["W_up"] = torch.stack([gen_slab(wl, "W_up", 0, g * G + hh, (d, wl.r)) for hh in range(G)])
    if wl.mode == "train":
        out["dO"] = torch.stack([gen_slab(wl, "dO", b, g * G + hh, (N, d)) for hh in range(G)])[None]
    if wl.needle != "none":
        _plant_group(wl, out, 0, 0, b, g)
    if dec:
        out["seq_len"] = torch.tensor([seq_lens(wl)[b]], dtype=torch.int32)
    return out


def segment_mean_query(wl: Workload, q: torch.Tensor, b: int, g: int, lo: int, hi: int) -> torch.Tensor:
    """Unit vector along the mean raw query of positions [lo, hi) over the
    group's heads, accumulated in fp64 (on the CPU, in a fixed order)."""
    acc = torch.zeros(wl.d, dtype=torch.float64)
    for h in range(g * wl.G, (g + 1) * wl.G):
        acc += q[b, h, lo:hi].to(torch.float64).cpu().sum(dim=0)
    return _unit(acc)


def needle_rows_for_oracle(wl: Workload, b: int, g: int):
    """Chunk ids planted in (b, g), for tests."""
    if wl.needle == "chunk7":
        return [7]
    if wl.needle == "segments":
        return needle_chunks_segments(wl, g)
    if wl.needle == "decode_random":
        return [needle_chunk_decode(wl, b, g)]
    return []


def slice_inputs(wl: Workload, t: dict, b: int, g: int) -> dict:
    """CPU copies of the (b, KV-group g) slabs an oracle needs for that group."""
    G = wl.G
    hs = slice(g * G, (g + 1) * G)
    out = dict(q=t["q"][b, hs].cpu(), k=t["k"][b, g].cpu(), v=t["v"][b, g].cpu(),
               kL=t["kL"][b, g].cpu(), e=t["e"][b, g].cpu())
    if "h" in t:
        out.update(h=t["h"][b].cpu(), W_down=t["W_down"][hs].cpu(), W_up=t["W_up"][hs].cpu())
    if "dO" in t:
        out["dO"] = t["dO"][b, hs].cpu()
    return out
