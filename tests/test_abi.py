"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point of include/hils.h, sizes workspaces and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import pytest

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
                r=32, qcal_shared=0, scale=0.0)
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


def test_fwd_strategy_switch():
    lib = L.lib()
    try:
        for s in (L.FWD_UNION, L.FWD_COMPACT, L.FWD_AUTO):
            assert lib.hils_set_fwd_strategy(s) == 0
        assert lib.hils_set_fwd_strategy(3) == 1 and lib.hils_set_fwd_strategy(-1) == 1
        # the forced strategy decides the LDS check: the 1.4B shape fits either way
        big = prob(B=1, Hq=32, Hkv=8, d=128, Nq=131072, Nk=131072, W=1024, D=2048)
        for s in (L.FWD_UNION, L.FWD_COMPACT):
            lib.hils_set_fwd_strategy(s)
            st, n = ws(big, L.OP_FWD)
            assert st in (0, 2), (s, st)
    finally:
        lib.hils_set_fwd_strategy(L.FWD_AUTO)


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
