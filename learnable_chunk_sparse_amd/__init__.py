"""HiLS attention for AMD Instinct MI355X: thin Python binding of libhils.so.

The functions here only marshal arguments: they allocate outputs and the
workspace with torch on the inputs' device, pass raw device pointers and the
current HIP stream to the C ABI (include/hils.h) and raise on a non-zero
status. Every step of the computation runs in the library's HIP kernels;
there is no fallback path. If libhils.so is missing, importing succeeds but
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhils.so")

HILS_FP32, HILS_BF16 = 0, 1
OP_ROUTE, OP_FWD, OP_BWD, OP_DECODE = 0, 1, 2, 3
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported problem",
          3: "workspace too small or misaligned", 4: "HIP launch failure"}

EXPORTS = ("hils_status_string", "hils_version", "hils_workspace_size", "hils_route",
           "hils_attn_fwd", "hils_attn_bwd", "hils_decode", "hils_decode_paged", "hils_landmark_fwd",
           "hils_landmark_bwd", "hils_hope", "hils_decode_noalloc", "hils_fwd_strategy_of")
NOALLOC_SCRATCH_BYTES = 64 << 20
FWD_AUTO, FWD_UNION, FWD_COMPACT, FWD_CHUNK_MAJOR = 0, 1, 2, 3
STEP_QCAL, STEP_ROUTE, STEP_ATTN_FWD, STEP_DECODE, STEP_BWD = 0, 1, 2, 3, 4
STEP_LANDMARK_FWD, STEP_LANDMARK_BWD, STEP_HOPE, STEP_WINDOW, STEP_CHUNKS = 5, 6, 7, 8, 9
STEP_PREP = 10
STEP_COUNT = 11


class HilsError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} (status {code})")
        self.code = code


class Timing(ctypes.Structure):
    """hils_timing: caller-owned (start, stop) event handles per step, one call."""
    _fields_ = [("start", ctypes.c_void_p * STEP_COUNT), ("stop", ctypes.c_void_p * STEP_COUNT)]


class Problem(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nk", ctypes.c_int32), ("S", ctypes.c_int32), ("K", ctypes.c_int32),
                ("W", ctypes.c_int32), ("D", ctypes.c_int32), ("r", ctypes.c_int32),
                ("qcal_shared", ctypes.c_int32), ("scale", ctypes.c_float),
                ("fwd_strategy", ctypes.c_int32), ("timing", ctypes.POINTER(Timing))]


class HopeParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32), ("base", ctypes.c_float),
                ("train_len", ctypes.c_int32), ("interleaved", ctypes.c_int32),
                ("inverse", ctypes.c_int32), ("timing", ctypes.POINTER(Timing))]


def make_timing(events) -> Optional[Timing]:
    """A Timing from {step: (start, stop)} of recorded torch.cuda.Event(enable_timing=True)
    (the events must have been recorded once so that their HIP handles exist);
    None for None or an empty dict."""
    if not events:
        return None
    tm = Timing()
    for step, (a, b) in events.items():
        if not 0 <= step < STEP_COUNT:
            raise ValueError(f"bad step id {step}")
        tm.start[step] = a.cuda_event
        tm.stop[step] = b.cuda_event
    return tm


def _attach(p, timing):
    """Point p.timing at a Timing built from `timing` (kept alive on p)."""
    tm = make_timing(timing) if isinstance(timing, dict) else timing
    if tm is not None:
        p._timing_keep = tm
        p.timing = ctypes.pointer(tm)
    return p


_lib = None


def lib():
    """The loaded library (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m learnable_chunk_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        P = ctypes.POINTER(Problem)
        L.hils_status_string.restype = ctypes.c_char_p
        L.hils_status_string.argtypes = [ctypes.c_int]
        L.hils_version.restype = i32
        L.hils_workspace_size.restype = ctypes.c_int
        L.hils_workspace_size.argtypes = [P, i32, ctypes.POINTER(sz)]
        L.hils_fwd_strategy_of.restype = ctypes.c_int
        L.hils_fwd_strategy_of.argtypes = [P, ctypes.POINTER(i32)]
        L.hils_route.restype = ctypes.c_int
        L.hils_route.argtypes = [P] + [vp] * 9 + [sz, vp]
        L.hils_attn_fwd.restype = ctypes.c_int
        L.hils_attn_fwd.argtypes = [P] + [vp] * 12 + [sz, vp]
        L.hils_attn_bwd.restype = ctypes.c_int
        L.hils_attn_bwd.argtypes = [P] + [vp] * 21 + [sz, vp]
        L.hils_decode.restype = ctypes.c_int
        L.hils_decode.argtypes = [P] + [vp] * 13 + [sz, vp]
        L.hils_decode_noalloc.restype = ctypes.c_int
        L.hils_decode_noalloc.argtypes = [P] + [vp] * 13
        L.hils_decode_paged.restype = ctypes.c_int
        L.hils_decode_paged.argtypes = [P, vp, vp, vp, vp, i32] + [vp] * 10 + [sz, vp]
        L.hils_landmark_fwd.restype = ctypes.c_int
        L.hils_landmark_fwd.argtypes = [P] + [vp] * 7
        L.hils_landmark_bwd.restype = ctypes.c_int
        L.hils_landmark_bwd.argtypes = [P] + [vp] * 7
        L.hils_hope.argtypes = [ctypes.POINTER(HopeParams), vp, vp, vp, vp]
        L.hils_hope.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HILS_BF16
    if t.dtype == torch.float32:
        return HILS_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _check(fn: str, code: int):
    if code != 0:
        raise HilsError(fn, code)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _validate(ref, specs):
    """Checks every tensor against (name, tensor, shape, dtype) before any
    pointer reaches the library: shape entries of None match any size, dtype
    "ref" means the dtype of `ref`; tensors given as None are skipped. Then
    every tensor must be a CUDA tensor on ref's device (a host pointer handed
    to a kernel would fault the GPU). Raises TypeError / ValueError."""
    if not isinstance(ref, torch.Tensor):
        raise TypeError("expected a torch tensor")
    _dtype_code(ref)
    if not ref.is_contiguous():
        raise ValueError("tensors must be contiguous")
    for name, t, shape, dt in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        want = ref.dtype if dt == "ref" else dt
        if t.dtype != want:
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
        if len(t.shape) != len(shape) or any(w is not None and w != g
                                             for w, g in zip(shape, t.shape)):
            raise ValueError(f"{name} must have shape {tuple('*' if w is None else w for w in shape)}, "
                             f"got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if ref.device.type != "cuda":
        raise ValueError("tensors must be on a CUDA (HIP) device")
    for name, t, _, _ in specs:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _qcal_specs(Hq, d, N, B, h, W_down, W_up, decode=False):
    """Shape specs of the Q-Cal inputs (all three or none)."""
    if (h is None) != (W_down is None) or (W_down is None) != (W_up is None):
        raise ValueError("h, W_down and W_up are given together (Q-Cal) or not at all")
    if W_down is None:
        return []
    D = h.shape[-1]
    r = W_down.shape[-2]
    if W_down.dim() == 2:
        wd, wu = (r, D), (d, r)
    else:
        wd, wu = (Hq, r, D), (Hq, d, r)
    hs = (B, D) if decode else (B, N, D)
    return [("h", h, hs, "ref"), ("W_down", W_down, wd, "ref"), ("W_up", W_up, wu, "ref")]


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _qcal_shared(W_down, Hq: int, D: int) -> int:
    """1 for one Q-Cal pair shared by all heads (W_down [r, D]), 0 for a pair
    per head (W_down [Hq, r, D]); any other shape is an error (the library
    reads the weights by these shapes)."""
    if W_down is None:
        return 0
    if W_down.dim() == 2 and W_down.shape[1] == D:
        return 1
    if W_down.dim() == 3 and W_down.shape[0] == Hq and W_down.shape[2] == D:
        return 0
    raise ValueError(f"W_down must be [Hq, r, D] or [r, D] (shared); got {tuple(W_down.shape)}")


def make_problem(q, k, S, K, W, h=None, W_down=None, scale=0.0, decode=False, strategy=0,
                 timing=None) -> Problem:
    B, Hq = q.shape[0], q.shape[1]
    d = q.shape[-1]
    Hkv = k.shape[1]
    Nk = k.shape[2]
    Nq = 1 if decode else q.shape[2]
    r = 0 if W_down is None else W_down.shape[-2]
    D = 0 if h is None else h.shape[-1]
    # W_down [r, D] (and W_up [d, r]): one Q-Cal pair shared by all heads
    shared = _qcal_shared(W_down, Hq, D)
    p = Problem(_dtype_code(q), B, Hq, Hkv, d, Nq, Nk, S, K, W, D, r, shared, float(scale),
                int(strategy), None)
    return _attach(p, timing)


def _prefill_specs(q, k, v, kL, e, S, h, W_down, W_up):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1] if k is not None and k.dim() == 4 else kL.shape[1]
    C = N // S
    return ([("k", k, (B, Hkv, N, d), "ref"), ("v", v, (B, Hkv, N, d), "ref"),
             ("kL", kL, (B, Hkv, C, d), "ref"), ("e", e, (B, Hkv, C), "ref")]
            + _qcal_specs(Hq, d, N, B, h, W_down, W_up))


def workspace_size(p: Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("hils_workspace_size", lib().hils_workspace_size(ctypes.byref(p), op, ctypes.byref(n)))
    return n.value


def fwd_strategy_of(p: Problem) -> int:
    """The forward strategy hils_attn_fwd runs for p (FWD_UNION, FWD_COMPACT
    or FWD_CHUNK_MAJOR)."""
    n = ctypes.c_int32(0)
    _check("hils_fwd_strategy_of", lib().hils_fwd_strategy_of(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def _workspace(p: Problem, op: int, device) -> torch.Tensor:
    n = workspace_size(p, op)
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def hils_route(q, kL, e, S: int, K: int, W: int, h=None, W_down=None, W_up=None, scale=0.0,
               with_scores=False, timing=None):
    """Top-K chunk selection. q [B,Hq,N,d]; kL [B,Hkv,C,d]; e [B,Hkv,C].
    Returns topk_idx [B,Hkv,N,K] int32 (and topk_score [B,Hq,N,K] fp32)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d]")
    _validate(q, _prefill_specs(q, None, None, kL, e, S, h, W_down, W_up))
    B, Hq, N, d = q.shape
    Hkv = kL.shape[1]
    fake_k = torch.empty((B, Hkv, N, 0), device=q.device)
    p = make_problem(q, fake_k, S, K, W, h, W_down, scale, timing=timing)
    dev = q.device
    idx = torch.empty((B, Hkv, N, K), dtype=torch.int32, device=dev)
    sc = torch.empty((B, Hq, N, K), dtype=torch.float32, device=dev) if with_scores else None
    ws = _workspace(p, OP_ROUTE, dev)
    _check("hils_route", lib().hils_route(ctypes.byref(p), _ptr(q), _ptr(kL), _ptr(e), _ptr(h),
                                          _ptr(W_down), _ptr(W_up), _ptr(idx), _ptr(sc), _ptr(ws),
                                          ws.numel(), _stream(dev)))
    return (idx, sc) if with_scores else idx


def hils_attn_fwd(q, k, v, kL, e, S: int, K: int, W: int, h=None, W_down=None, W_up=None,
                  scale=0.0, out=None, strategy=FWD_AUTO, timing=None):
    """Prefill forward. Returns (o [B,Hq,N,d], lse [B,Hq,N] fp32, topk_idx [B,Hkv,N,K]).
    strategy: FWD_AUTO, FWD_UNION, FWD_COMPACT or FWD_CHUNK_MAJOR (same result);
    timing: {step: (start_event, stop_event)} recorded around that step's launches."""
    if q.dim() != 4 or k is None or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k [B, Hkv, N, d]")
    _validate(q, _prefill_specs(q, k, v, kL, e, S, h, W_down, W_up))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    p = make_problem(q, k, S, K, W, h, W_down, scale, strategy=strategy, timing=timing)
    dev = q.device
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        idx = torch.empty((B, Hkv, N, K), dtype=torch.int32, device=dev)
        ws = _workspace(p, OP_FWD, dev)
    else:
        o, lse, idx, ws = out
        _validate(q, [("o", o, tuple(q.shape), "ref"), ("lse", lse, (B, Hq, N), torch.float32),
                      ("topk_idx", idx, (B, Hkv, N, K), torch.int32),
                      ("workspace", ws, (None,), torch.uint8)])
    _check("hils_attn_fwd", lib().hils_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kL),
                                                _ptr(e), _ptr(h), _ptr(W_down), _ptr(W_up), _ptr(o),
                                                _ptr(lse), _ptr(idx), _ptr(ws), ws.numel(),
                                                _stream(dev)))
    return o, lse, idx


def fwd_buffers(q, k, S, K, W, h=None, W_down=None, scale=0.0, strategy=FWD_AUTO):
    """Preallocated (o, lse, topk_idx, workspace) for repeated hils_attn_fwd calls."""
    B, Hq, N, d = q.shape
    p = make_problem(q, k, S, K, W, h, W_down, scale, strategy=strategy)
    dev = q.device
    return (torch.empty_like(q), torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
            torch.empty((B, k.shape[1], N, K), dtype=torch.int32, device=dev),
            _workspace(p, OP_FWD, dev))


def hils_attn_bwd(q, k, v, kL, e, o, lse, topk_idx, dO, S: int, K: int, W: int, h=None, W_down=None,
                  W_up=None, scale=0.0, want_dh=False, out=None, timing=None):
    """Backward with the forward's selection held fixed. Returns a dict of fp32
    gradients dq, dk, dv, dkL, de (+ dW_down, dW_up, dh with Q-Cal)."""
    if q.dim() != 4 or k is None or k.dim() != 4:
        raise ValueError("q must be [B, Hq, N, d] and k [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _validate(q, _prefill_specs(q, k, v, kL, e, S, h, W_down, W_up) + [
        ("o", o, (B, Hq, N, d), "ref"), ("lse", lse, (B, Hq, N), torch.float32),
        ("topk_idx", topk_idx, (B, Hkv, N, K), torch.int32), ("dO", dO, (B, Hq, N, d), "ref")])
    if lse is None or topk_idx is None or dO is None:
        raise ValueError("lse, topk_idx and dO are required")
    p = make_problem(q, k, S, K, W, h, W_down, scale, timing=timing)
    dev = q.device
    f = dict(dtype=torch.float32, device=dev)
    if out is None:
        g = dict(dq=torch.empty(q.shape, **f), dk=torch.empty(k.shape, **f),
                 dv=torch.empty(v.shape, **f), dkL=torch.empty(kL.shape, **f),
                 de=torch.empty(e.shape, **f))
        if W_down is not None:
            g["dW_down"] = torch.empty(W_down.shape, **f)
            g["dW_up"] = torch.empty(W_up.shape, **f)
            if want_dh:
                g["dh"] = torch.empty(h.shape, **f)
        ws = _workspace(p, OP_BWD, dev)
    else:
        g, ws = out
    _check("hils_attn_bwd", lib().hils_attn_bwd(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kL), _ptr(e), _ptr(h), _ptr(W_down),
        _ptr(W_up), _ptr(o), _ptr(lse), _ptr(topk_idx), _ptr(dO), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g["dkL"]), _ptr(g["de"]), _ptr(g.get("dW_down")), _ptr(g.get("dW_up")),
        _ptr(g.get("dh")), _ptr(ws), ws.numel(), _stream(dev)))
    return g


def _decode_specs(q, k_cache, v_cache, kL, e, S, seq_len, h, W_down, W_up):
    if q.dim() != 3 or k_cache is None or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, Hkv, Nk, d]")
    B, Hq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    C = Nk // S
    return ([("k_cache", k_cache, (B, Hkv, Nk, d), "ref"), ("v_cache", v_cache, (B, Hkv, Nk, d), "ref"),
             ("kL", kL, (B, Hkv, C, d), "ref"), ("e", e, (B, Hkv, C), "ref"),
             ("seq_len", seq_len, (B,), torch.int32)]
            + _qcal_specs(Hq, d, 1, B, h, W_down, W_up, decode=True))


def hils_decode(q, k_cache, v_cache, kL, e, S: int, K: int, W: int, seq_len=None, h=None,
                W_down=None, W_up=None, scale=0.0, out=None, with_topk=True, timing=None):
    """One decode step. q [B,Hq,d]; caches [B,Hkv,Nk,d]; seq_len [B] int32 (device).
    Returns (o [B,Hq,d], lse [B,Hq], topk_idx [B,Hkv,K] or None)."""
    _validate(q, _decode_specs(q, k_cache, v_cache, kL, e, S, seq_len, h, W_down, W_up))
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    p = make_problem(q, k_cache, S, K, W, h, W_down, scale, decode=True, timing=timing)
    dev = q.device
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        idx = torch.empty((B, Hkv, K), dtype=torch.int32, device=dev) if with_topk else None
        ws = _workspace(p, OP_DECODE, dev)
    else:
        o, lse, idx, ws = out
    _check("hils_decode", lib().hils_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(seq_len), _ptr(kL), _ptr(e), _ptr(h), _ptr(W_down),
                                            _ptr(W_up), _ptr(o), _ptr(lse), _ptr(idx), _ptr(ws),
                                            ws.numel(), _stream(dev)))
    return o, lse, idx


def hils_decode_noalloc(q, k_cache, v_cache, kL, e, S: int, K: int, W: int, seq_len=None, h=None,
                        W_down=None, W_up=None, scale=0.0, out=None, with_topk=True, timing=None):
    """hils_decode on the library's static per-GPU scratch (no workspace, no
    device allocation inside the call; pass `out` = (o, lse, topk_idx or None)
    to allocate nothing at all). Calls on one GPU must not overlap."""
    _validate(q, _decode_specs(q, k_cache, v_cache, kL, e, S, seq_len, h, W_down, W_up))
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    p = make_problem(q, k_cache, S, K, W, h, W_down, scale, decode=True, timing=timing)
    dev = q.device
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        idx = torch.empty((B, Hkv, K), dtype=torch.int32, device=dev) if with_topk else None
    else:
        o, lse, idx = out
        _validate(q, [("o", o, tuple(q.shape), "ref"), ("lse", lse, (B, Hq), torch.float32),
                      ("topk_idx", idx, (B, Hkv, K), torch.int32)])
    _check("hils_decode_noalloc", lib().hils_decode_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_len), _ptr(kL), _ptr(e),
        _ptr(h), _ptr(W_down), _ptr(W_up), _ptr(o), _ptr(lse), _ptr(idx), _stream(dev)))
    return o, lse, idx


def hils_decode_paged(q, k_pages, v_pages, page_table, seq_len, kL_pages, e_pages, S: int, K: int,
                      W: int, h=None, W_down=None, W_up=None, scale=0.0, out=None, with_topk=True,
                      timing=None):
    """One decode step over a paged cache: k_pages / v_pages [P, Hkv, S, d],
    kL_pages [P, Hkv, d], e_pages [P, Hkv], page_table [B, max_pages] int32
    (page of each chunk), seq_len [B] int32 (device). Returns (o, lse,
    topk_idx or None) as hils_decode."""
    if q.dim() != 3 or k_pages is None or k_pages.dim() != 4 or page_table is None:
        raise ValueError("q [B, Hq, d], pages [P, Hkv, S, d] and page_table are required")
    B, Hq, d = q.shape
    P, Hkv = k_pages.shape[0], k_pages.shape[1]
    _validate(q, [("k_pages", k_pages, (P, Hkv, S, d), "ref"), ("v_pages", v_pages, (P, Hkv, S, d), "ref"),
                  ("page_table", page_table, (B, None), torch.int32),
                  ("seq_len", seq_len, (B,), torch.int32),
                  ("kL_pages", kL_pages, (P, Hkv, d), "ref"), ("e_pages", e_pages, (P, Hkv), "ref")]
              + _qcal_specs(Hq, d, 1, B, h, W_down, W_up, decode=True))
    if seq_len is None:
        raise ValueError("seq_len is required for a paged cache")
    max_pages = page_table.shape[1]
    r = 0 if W_down is None else W_down.shape[-2]
    D = 0 if h is None else h.shape[-1]
    p = _attach(Problem(_dtype_code(q), B, Hq, Hkv, d, 1, max_pages * S, S, K, W, D, r,
                        _qcal_shared(W_down, Hq, D), float(scale), 0, None), timing)
    dev = q.device
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        idx = torch.empty((B, Hkv, K), dtype=torch.int32, device=dev) if with_topk else None
        ws = _workspace(p, OP_DECODE, dev)
    else:
        o, lse, idx, ws = out
    _check("hils_decode_paged", lib().hils_decode_paged(
        ctypes.byref(p), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), max_pages,
        _ptr(seq_len), _ptr(kL_pages), _ptr(e_pages), _ptr(h), _ptr(W_down), _ptr(W_up), _ptr(o),
        _ptr(lse), _ptr(idx), _ptr(ws), ws.numel(), _stream(dev)))
    return o, lse, idx


def decode_buffers(q, k_cache, S, K, W, h=None, W_down=None, scale=0.0):
    B, Hq, d = q.shape
    p = make_problem(q, k_cache, S, K, W, h, W_down, scale, decode=True)
    dev = q.device
    return (torch.empty_like(q), torch.empty((B, Hq), dtype=torch.float32, device=dev),
            torch.empty((B, k_cache.shape[1], K), dtype=torch.int32, device=dev),
            _workspace(p, OP_DECODE, dev))


def _landmark_problem(qL, k, S, scale, timing=None) -> Problem:
    if qL.dim() != 4 or k is None or k.dim() != 4:
        raise ValueError("qL must be [B, Hkv, C, d] and k [B, Hkv, N, d]")
    B, Hkv, C, d = qL.shape
    if k.shape[0] != B or k.shape[1] != Hkv or k.shape[3] != d or k.dtype != qL.dtype:
        raise ValueError("qL [B, Hkv, C, d] and k [B, Hkv, N, d] must agree")
    if C != k.shape[2] // S:
        raise ValueError("qL needs one landmark query per complete chunk (C = N // S)")
    _validate(qL, [("k", k, tuple(k.shape), "ref")])
    return _attach(Problem(_dtype_code(qL), B, Hkv, Hkv, d, k.shape[2], k.shape[2], S, 1, 1, 0, 0, 0,
                           float(scale), 0, None), timing)


def hils_landmark_fwd(qL, k, S: int, scale=0.0, want_f32=False, timing=None):
    """Landmark key kL [B, Hkv, C, d] and entropy bias e [B, Hkv, C] of every
    complete chunk from its landmark query qL (dtype of qL); with want_f32 also
    their fp32 values: returns (kL, e) or (kL, e, kL32, e32)."""
    p = _landmark_problem(qL, k, S, scale, timing)
    dev = qL.device
    kL = torch.empty(qL.shape, dtype=qL.dtype, device=dev)
    e = torch.empty(qL.shape[:3], dtype=qL.dtype, device=dev)
    kL32 = torch.empty(qL.shape, dtype=torch.float32, device=dev) if want_f32 else None
    e32 = torch.empty(qL.shape[:3], dtype=torch.float32, device=dev) if want_f32 else None
    _check("hils_landmark_fwd", lib().hils_landmark_fwd(ctypes.byref(p), _ptr(qL), _ptr(k), _ptr(kL),
                                                        _ptr(e), _ptr(kL32), _ptr(e32), _stream(dev)))
    return (kL, e, kL32, e32) if want_f32 else (kL, e)


def hils_landmark_bwd(qL, k, dkL, de, S: int, dk=None, scale=0.0, timing=None):
    """Gradients of the landmark summary: returns (dqL, dk) with dqL fp32
    [B, Hkv, C, d]; the keys' part is ADDED into dk (fp32 [B, Hkv, N, d],
    zero-initialised when not given)."""
    p = _landmark_problem(qL, k, S, scale, timing)
    dev = qL.device
    _validate(qL, [("dkL", dkL, tuple(qL.shape), torch.float32),
                   ("de", de, tuple(qL.shape[:3]), torch.float32),
                   ("dk", dk, tuple(k.shape), torch.float32)])
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    dqL = torch.empty(qL.shape, dtype=torch.float32, device=dev)
    _check("hils_landmark_bwd", lib().hils_landmark_bwd(ctypes.byref(p), _ptr(qL), _ptr(k), _ptr(dkL),
                                                        _ptr(de), _ptr(dqL), _ptr(dk), _stream(dev)))
    return dqL, dk


def hils_hope(x, pos=None, base: float = 10000.0, train_len: int = 8192, interleaved=False,
              inverse=False, out=None, timing=None):
    """HoPE rotation of x [B, H, N, d] (bf16 or fp32): the rotary pairs whose
    period 2 pi base^(2j/d) fits train_len turn by pos * theta_j (by minus
    that when inverse, the transpose used for gradients); the other pairs are
    copied. pos: int32 [B, N] or None (position n). out may be x (in place);
    returns out."""
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    _validate(x, [("pos", pos, (B, N), torch.int32), ("out", out, tuple(x.shape), "ref")])
    if out is None:
        out = torch.empty_like(x)
    p = HopeParams(_dtype_code(x), B, H, N, d, float(base), int(train_len), int(bool(interleaved)),
                   int(bool(inverse)), None)
    tm = make_timing(timing) if isinstance(timing, dict) else timing
    if tm is not None:
        p.timing = ctypes.pointer(tm)
    _check("hils_hope", lib().hils_hope(ctypes.byref(p), _ptr(x), _ptr(out), _ptr(pos),
                                        _stream(x.device)))
    return out
