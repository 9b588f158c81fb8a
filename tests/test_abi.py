"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point of include/hils.h, sizes workspaces and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import pytest
import torch

import learnable_chunk_sparse_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "hils.h")).read()
    return sorted(set(re.findall(r"\b(hils_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = header_functions()
    assert {"hils_attn_fwd", "hils_attn_bwd", "hils_decode", "hils_route"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(L.EXPORTS) == set(names)


def prob(**kw):
    base = dict(dtype=1, B=4, Hq=16, Hkv=16, d=64, Nq=8192, Nk=8192, S=64, K=16, W=512, D=1024,
                r=32, qcal_shared=0, scale=0.0, fwd_strategy=0, timing=None)
    base.update(kw)
    return L.Problem(*[base[f[0]] for f in L.Problem._fields_])


def ws(p, op):
    n = ctypes.c_size_t(0)
    st = L.lib().hils_workspace_size(ctypes.byref(p), op, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes():
    st, n = ws(prob(), L.OP_FWD)
    assert st == 0
    rows = 4 * 16 * 8192
    assert n >= rows * 64 * 4 + rows * 16 * 4  # fp32 q_hat + selected scores
    st, n2 = ws(prob(r=0, D=0), L.OP_FWD)
    assert st == 0 and n2 < n


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), 1), (dict(B=0), 1), (dict(K=0), 1), (dict(Nq=100, Nk=200), 1),
    (dict(d=96), 2), (dict(S=32), 2), (dict(dtype=7), 2), (dict(qcal_shared=2), 1),
    (dict(r=8), 2), (dict(Hq=16, Hkv=1), 2), (dict(scale=-1.0), 1),
])
def test_validation_codes(kw, code):
    st, _ = ws(prob(**kw), L.OP_FWD)
    assert st == code, (kw, st)


def test_shared_qcal_workspace_holds_the_per_head_copies():
    """qcal_shared = 1: each op's workspace grows by the per-head copies of the
    pair (and, for the backward, the per-head weight gradients)."""
    Hq, r, D, d = 16, 32, 1024, 64
    for op, extra in [(L.OP_ROUTE, 2 * Hq * (r * D + d * r)), (L.OP_FWD, 2 * Hq * (r * D + d * r)),
                      (L.OP_BWD, (2 + 4) * Hq * (r * D + d * r))]:
        st0, n0 = ws(prob(), op)
        st1, n1 = ws(prob(qcal_shared=1), op)
        assert st0 == 0 and st1 == 0
        assert extra <= n1 - n0 <= extra + 4 * 256, (op, n1 - n0, extra)
        st2, n2 = ws(prob(qcal_shared=1, r=0, D=0), op)
        st3, n3 = ws(prob(r=0, D=0), op)
        assert n2 == n3  # no Q-Cal: nothing shared


def test_fp32_d128_backward_has_a_workspace():
    st, nbytes = ws(prob(dtype=0, d=128), L.OP_BWD)
    assert st == 0 and nbytes > 0


def test_calls_reject_before_launch():
    lib = L.lib()
    p = prob()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    # missing required pointer
    st = lib.hils_attn_fwd(ctypes.byref(p), null, fake, fake, fake, fake, fake, fake, fake, fake,
                           fake, fake, fake, 1 << 40, null)
    assert st == 1
    # workspace too small
    st = lib.hils_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                           fake, fake, ctypes.c_void_p(4096), 16, null)
    assert st == 3
    # misaligned workspace
    st = lib.hils_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                           fake, fake, ctypes.c_void_p(4096 + 8), 1 << 40, null)
    assert st == 3
    # decode needs Nq == 1
    st = lib.hils_decode(ctypes.byref(p), fake, fake, fake, null, fake, fake, fake, fake, fake, fake,
                         fake, null, fake, 1 << 40, null)
    assert st == 1
    assert lib.hils_status_string(3) == b"workspace too small or misaligned"


def test_landmark_calls_reject_before_launch():
    """The landmark entry points validate their own fields (Hq, K, W, r are
    not read) and return before any launch."""
    lib = L.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    ok = prob(Hq=3, K=0, W=0, r=5, D=0)  # fields the landmark ops ignore
    assert lib.hils_landmark_fwd(ctypes.byref(ok), null, fake, fake, fake, null, null, null) == 1
    assert lib.hils_landmark_fwd(ctypes.byref(ok), fake, fake, fake, null, null, null, null) == 1
    assert lib.hils_landmark_bwd(ctypes.byref(ok), fake, fake, fake, fake, fake, null, null) == 1
    odd = ctypes.c_void_p(0x1004)  # rows move as 16-byte vectors
    assert lib.hils_landmark_fwd(ctypes.byref(ok), odd, fake, fake, fake, null, null, null) == 1
    assert lib.hils_landmark_fwd(ctypes.byref(ok), fake, fake, fake, fake, odd, null, null) == 1
    assert lib.hils_landmark_bwd(ctypes.byref(ok), fake, fake, fake, fake, fake, odd, null) == 1
    for kw, code in [(dict(d=96), 2), (dict(S=32), 2), (dict(B=0), 1), (dict(Nk=0), 1),
                     (dict(scale=float("inf")), 1), (dict(dtype=5), 2)]:
        p = prob(**kw)
        assert lib.hils_landmark_fwd(ctypes.byref(p), fake, fake, fake, fake, null, null, null) == code, kw
        assert lib.hils_landmark_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, null) == code, kw


def test_hope_rejects_before_launch_and_empty_is_a_no_op():
    """hils_hope validates its parameters and returns before any launch; an
    empty tensor (B, H or N == 0) is a successful no-op."""
    lib = L.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)

    def hp(**kw):
        f = dict(dtype=1, B=2, H=4, N=100, d=64, base=1e4, train_len=8192, interleaved=0, inverse=0)
        f.update(kw)
        return L.HopeParams(**f)

    assert lib.hils_hope(None, fake, fake, null, null) == 1
    assert lib.hils_hope(ctypes.byref(hp()), null, fake, null, null) == 1
    assert lib.hils_hope(ctypes.byref(hp()), fake, null, null, null) == 1
    assert lib.hils_hope(ctypes.byref(hp()), ctypes.c_void_p(0x1008), fake, null, null) == 1
    for kw, code in [(dict(d=96), 2), (dict(d=32), 2), (dict(dtype=3), 1), (dict(B=-1), 1),
                     (dict(base=1.0), 1), (dict(base=float("nan")), 1), (dict(train_len=-5), 1),
                     (dict(interleaved=2), 1), (dict(inverse=-1), 1),
                     (dict(B=1 << 20, N=1 << 20), 1)]:
        assert lib.hils_hope(ctypes.byref(hp(**kw)), fake, fake, null, null) == code, kw
    for kw in (dict(B=0), dict(H=0), dict(N=0)):
        assert lib.hils_hope(ctypes.byref(hp(**kw)), fake, fake, null, null) == 0, kw
        assert lib.hils_hope(ctypes.byref(hp(**kw)), null, null, null, null) == 0, kw


def test_fwd_strategy_is_a_field_of_the_call():
    """The forward strategy travels in the problem (no process-wide switch):
    the workspace size is computed for the strategy the call names, and
    values outside the enum are rejected."""
    assert not hasattr(L.lib(), "hils_set_fwd_strategy")
    assert not hasattr(L.lib(), "hils_set_timing_events")
    for s_ in (L.FWD_AUTO, L.FWD_UNION, L.FWD_COMPACT):
        st, _ = ws(prob(fwd_strategy=s_), L.OP_FWD)
        assert st == 0, s_
    for bad in (-1, 4):
        assert ws(prob(fwd_strategy=bad), L.OP_FWD)[0] == 1
    # the strategy decides the LDS check: the 1.4B shape fits either way
    big = prob(B=1, Hq=32, Hkv=8, d=128, Nq=131072, Nk=131072, W=1024, D=2048)
    for s_ in (L.FWD_UNION, L.FWD_COMPACT):
        big.fwd_strategy = s_
        st, n = ws(big, L.OP_FWD)
        assert st in (0, 2), (s_, st)


def test_fwd_strategy_of_reports_what_the_call_runs():
    """hils_fwd_strategy_of returns the problem's own strategy when it names
    one and resolves AUTO by shape: packed union where a tile's selections
    cover the chunks several times over (the 345M prefill), chunk-major for
    the long GQA prefills (131072 and 524288 tokens); errors as the forward's
    workspace query."""
    for s_ in (L.FWD_UNION, L.FWD_COMPACT, L.FWD_CHUNK_MAJOR):
        assert L.fwd_strategy_of(prob(fwd_strategy=s_)) == s_
    assert L.fwd_strategy_of(prob()) == L.FWD_UNION
    big = prob(B=1, Hq=32, Hkv=8, d=128, Nq=131072, Nk=131072, W=1024, D=2048)
    assert L.fwd_strategy_of(big) == L.FWD_CHUNK_MAJOR
    long_ = prob(B=1, Nq=524288, Nk=524288, K=32, r=0, D=0)
    assert L.fwd_strategy_of(long_) == L.FWD_CHUNK_MAJOR
    out = ctypes.c_int32(-7)
    lib = L.lib()
    assert lib.hils_fwd_strategy_of(ctypes.byref(prob(Hq=6, Hkv=4)), ctypes.byref(out)) == 1
    assert lib.hils_fwd_strategy_of(ctypes.byref(prob(d=96)), ctypes.byref(out)) == 2
    assert lib.hils_fwd_strategy_of(ctypes.byref(prob()), None) == 1
    assert out.value == -7  # nothing written on error


def test_timing_struct_layout():
    """hils_timing is STEP_COUNT start handles then STEP_COUNT stop handles,
    and the problem carries a pointer to it after the strategy field."""
    assert ctypes.sizeof(L.Timing) == 2 * L.STEP_COUNT * ctypes.sizeof(ctypes.c_void_p)
    assert L.Problem.timing.offset % ctypes.sizeof(ctypes.c_void_p) == 0
    assert L.Problem.fwd_strategy.offset == 14 * 4
    tm = L.Timing()
    p = prob(timing=ctypes.pointer(tm))
    assert ws(p, L.OP_FWD)[0] == 0  # sizing reads no events


def test_decode_paged_rejects_before_launch():
    lib = L.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    p = prob(Nq=1, Nk=64 * 100, r=0, D=0)
    args = lambda pt, mp, sl, wsb: (ctypes.byref(p), fake, fake, fake, pt, mp, sl, fake, fake, null,
                                    null, null, fake, fake, null, fake, wsb, null)
    assert lib.hils_decode_paged(*args(null, 100, fake, 1 << 40)) == 1  # no page table
    assert lib.hils_decode_paged(*args(fake, 100, null, 1 << 40)) == 1  # no seq_len
    assert lib.hils_decode_paged(*args(fake, 99, fake, 1 << 40)) == 1   # max_pages * S != Nk
    assert lib.hils_decode_paged(*args(fake, 100, fake, 16)) == 3       # workspace too small


def test_chunk_tensors_may_be_null_only_without_complete_chunks():
    lib = L.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    for Nk, code in [(50, 3), (8192, 1)]:  # 3: passed validation, then the workspace check
        p = prob(Nq=Nk, Nk=Nk, r=0, D=0)
        st = lib.hils_attn_fwd(ctypes.byref(p), fake, fake, fake, null, null, null, null, null, fake,
                               fake, fake, fake, 16, null)
        assert st == code, (Nk, st)


# ---------------------------------------------------------------- binding argument checks
def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _fwd_args(**over):
    B, Hq, Hkv, N, d, S = 1, 4, 2, 256, 64, 64
    a = dict(q=_t(B, Hq, N, d), k=_t(B, Hkv, N, d), v=_t(B, Hkv, N, d), kL=_t(B, Hkv, N // S, d),
             e=_t(B, Hkv, N // S))
    a.update(over)
    return a


@pytest.mark.parametrize("over,exc", [
    (dict(k=_t(1, 2, 256, 64, dtype=torch.float32)), TypeError),       # k dtype != q dtype
    (dict(v=_t(1, 2, 255, 64)), ValueError),                           # v shape
    (dict(kL=_t(1, 2, 3, 64)), ValueError),                            # wrong chunk count
    (dict(e=_t(1, 2, 4, dtype=torch.float32)), TypeError),             # e dtype
    (dict(q=_t(1, 4, 256, 64, dtype=torch.float16)), TypeError),       # unsupported dtype
    (dict(kL=_t(1, 2, 64, 4).transpose(2, 3)), ValueError),           # not contiguous
    ({}, ValueError),                                                  # host tensors
])
def test_binding_rejects_bad_prefill_arguments(over, exc):
    a = _fwd_args(**over)
    with pytest.raises(exc):
        L.hils_attn_fwd(a["q"], a["k"], a["v"], a["kL"], a["e"], 64, 2, 64)


def test_binding_rejects_bad_qcal_and_backward_arguments():
    a = _fwd_args()
    h, Wd, Wu = _t(1, 256, 128), _t(4, 32, 128), _t(4, 64, 32)
    with pytest.raises(ValueError):  # Q-Cal tensors come together
        L.hils_attn_fwd(a["q"], a["k"], a["v"], a["kL"], a["e"], 64, 2, 64, h=h, W_down=Wd)
    with pytest.raises(TypeError):  # W_up dtype
        L.hils_attn_fwd(a["q"], a["k"], a["v"], a["kL"], a["e"], 64, 2, 64, h=h, W_down=Wd,
                        W_up=Wu.float())
    with pytest.raises(ValueError):  # W_up shape
        L.hils_attn_fwd(a["q"], a["k"], a["v"], a["kL"], a["e"], 64, 2, 64, h=h, W_down=Wd,
                        W_up=_t(4, 64, 16))
    lse, idx, dO = _t(1, 4, 256, dtype=torch.float32), _t(1, 2, 256, 2, dtype=torch.int32), _t(1, 4, 256, 64)
    with pytest.raises(TypeError):  # int64 selection
        L.hils_attn_bwd(a["q"], a["k"], a["v"], a["kL"], a["e"], None, lse, idx.long(), dO, 64, 2, 64)
    with pytest.raises(ValueError):  # K of topk_idx
        L.hils_attn_bwd(a["q"], a["k"], a["v"], a["kL"], a["e"], None, lse, idx, dO, 64, 3, 64)
    with pytest.raises(ValueError):  # host tensors
        L.hils_attn_bwd(a["q"], a["k"], a["v"], a["kL"], a["e"], None, lse, idx, dO, 64, 2, 64)


def test_binding_rejects_bad_decode_arguments():
    q = _t(2, 4, 64)
    kc = _t(2, 2, 640, 64)
    kL, e = _t(2, 2, 10, 64), _t(2, 2, 10)
    with pytest.raises(TypeError):  # int64 seq_len would be read as int32 halves
        L.hils_decode(q, kc, kc, kL, e, 64, 4, 128, seq_len=torch.tensor([640, 600]))
    with pytest.raises(ValueError):  # seq_len length
        L.hils_decode(q, kc, kc, kL, e, 64, 4, 128, seq_len=torch.tensor([640], dtype=torch.int32))
    with pytest.raises(ValueError):  # landmark count
        L.hils_decode(q, kc, kc, _t(2, 2, 9, 64), e, 64, 4, 128)
    with pytest.raises(ValueError):  # host tensors
        L.hils_decode(q, kc, kc, kL, e, 64, 4, 128, seq_len=torch.tensor([640, 600], dtype=torch.int32))


def test_decode_noalloc_rejects_oversize_and_invalid_before_touching_the_device():
    """The static-scratch decode sizes the problem first: a problem whose
    decode workspace exceeds the static buffer is refused with
    HILS_ERR_WORKSPACE, an invalid one with its validation code, both without
    any device call (this runs with no GPU)."""
    lib = L.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    small = prob(B=2, Hq=4, Hkv=2, d=64, Nq=1, Nk=4096, K=8, W=256, r=0, D=0)
    st, need = ws(small, L.OP_DECODE)
    assert st == 0 and need <= L.NOALLOC_SCRATCH_BYTES
    big = prob(B=256, Hq=64, Hkv=8, d=128, Nq=1, Nk=1 << 20, K=64, W=2048, r=0, D=0)
    st, need = ws(big, L.OP_DECODE)
    assert st == 0 and need > L.NOALLOC_SCRATCH_BYTES
    args = lambda p: (ctypes.byref(p), fake, fake, fake, null, fake, fake, null, null, null, fake,
                      fake, null, null)
    assert lib.hils_decode_noalloc(*args(big)) == 3
    assert lib.hils_decode_noalloc(*args(prob(B=0, Nq=1, Nk=4096))) == 1
    assert lib.hils_decode_noalloc(*args(prob(d=96, Nq=1, Nk=4096))) == 2


def test_forward_and_backward_accept_the_same_problems():
    """hils_workspace_size answers alike for the forward and the backward on a
    grid of shapes (head dims, GQA groups, K, dtypes, 8K to 2M tokens), with
    the default strategy and the chunk-major one: a problem the forward runs
    can be trained."""
    seen_ok = seen_bad = 0
    for d in (64, 128):
        for G in (1, 2, 4):
            for K in (8, 16, 32):
                for dt in (0, 1):
                    for N in (8192, 131072, 262144, 524288, 1048576, 2097152):
                        for strat in (L.FWD_AUTO, L.FWD_CHUNK_MAJOR):
                            p = prob(dtype=dt, B=1, Hq=8 * G, Hkv=8, d=d, Nq=N, Nk=N, K=K, W=512,
                                     r=0, D=0, fwd_strategy=strat)
                            f, _ = ws(p, L.OP_FWD)
                            b, _ = ws(p, L.OP_BWD)
                            assert (f == 0) == (b == 0), (d, G, K, dt, N, strat, f, b)
                            seen_ok += f == 0
                            seen_bad += f != 0
    assert seen_ok > 0 and seen_bad > 0
    # the paper's long-context prefill shape (345M: 16 heads, d 64, top-32, 512K tokens)
    p = prob(B=1, Hq=16, Hkv=16, d=64, Nq=524288, Nk=524288, K=32, W=512, D=1024, r=32)
    assert ws(p, L.OP_FWD)[0] == 0 and ws(p, L.OP_BWD)[0] == 0
