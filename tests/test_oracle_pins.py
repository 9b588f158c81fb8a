"""Pins for the fp64 oracle: each checks it against something other than
itself (a value printed on the pages, a closed form, a textbook routine, an
invariant of the method, or brute force on tiny inputs)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def small_inputs(seed=0, B=1, Hq=2, Hkv=1, N=64, d=8, S=4, D=6, r=3, qcal=True, e_shift=0.0):
    rng = np.random.default_rng(seed)
    C = N // S
    t = dict(q=rng.standard_normal((B, Hq, N, d)), k=rng.standard_normal((B, Hkv, N, d)),
             v=rng.standard_normal((B, Hkv, N, d)), kL=rng.standard_normal((B, Hkv, C, d)),
             e=rng.uniform(-1, 1, (B, Hkv, C)) + e_shift)
    if qcal:
        t.update(h=rng.standard_normal((B, N, D)), W_down=rng.standard_normal((Hq, r, D)) * 0.3,
                 W_up=rng.standard_normal((Hq, d, r)) * 0.3)
    return t


def full_causal_attention(q, k, v, scale):
    """Textbook causal softmax attention via torch SDPA in float64 on the CPU."""
    Q = torch.tensor(q)[None, None]
    Kt = torch.tensor(k)[None, None]
    Vt = torch.tensor(v)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True, scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- worked example
def test_qcal_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLD, "qcal_worked_example.json")))
    q = np.array(g["q"])[None]
    W_down = np.array(g["W_down"])[None]
    W_up = np.array(g["W_up"])[None]
    q_hat, u = H.qcal(q, np.array(g["h"]), W_down, W_up)
    np.testing.assert_allclose(q_hat[0] - q[0], g["expect_delta_q"], atol=1e-15)
    np.testing.assert_allclose(q_hat[0], g["expect_q_hat"], atol=1e-15)
    kL = np.array(g["k_landmark"])[None]
    np.testing.assert_allclose(q_hat[0] @ kL[0], g["expect_dot"], atol=1e-15)
    # the oracle's scoring step (row_forward, one distant chunk) must give 0.06
    d = g["d"]
    S, W = 1, 1
    i = 1  # query at position 1 with chunk 0 (token 0) distant
    K = np.zeros((2, d))
    r = H.row_forward(q, q_hat, K, K, kL, np.array([g["bias"]]), i, S, 1, W, 1 / math.sqrt(d))
    assert H.n_distant(i, W, S) == 1
    np.testing.assert_allclose(r.s[0, 0], g["expect_score"], atol=1e-15)


# ---------------------------------------------------------------- chunk geometry
@pytest.mark.parametrize("W,S", [(128, 64), (512, 64), (6, 4), (1, 1), (7, 3)])
def test_distant_chunks_and_window_partition(W, S):
    for i in range(0, 5 * (W + S)):
        nd = H.n_distant(i, W, S)
        # every distant chunk's newest token is at least W older than i
        for c in range(nd):
            assert c * S + S - 1 <= i - W
        # the next chunk is not distant
        assert not ((nd) * S + S - 1 <= i - W)
        ws = H.window_start(i, W, S)
        # window spans W .. W+S-1 tokens (or everything up to i early on)
        n_w = i + 1 - ws
        assert n_w >= min(W, i + 1) and n_w <= W + S - 1


# ---------------------------------------------------------------- top-K
def test_topk_matches_rank_count_definition():
    rng = np.random.default_rng(3)
    for trial in range(300):
        n = int(rng.integers(0, 40))
        sel = rng.integers(-3, 4, n).astype(float) if trial % 2 else rng.standard_normal(n)
        k = int(rng.integers(0, n + 2))
        got = list(H.select_topk(sel, min(k, n)))
        ref = brute.rank_count_topk(list(sel), min(k, n))
        assert got == ref


def test_topk_matches_subset_enumeration():
    """The selected set is the unique k-subset whose every member precedes
    every non-member in (score desc, index asc) order."""
    rng = np.random.default_rng(4)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        sel = rng.integers(-2, 3, n).astype(float)
        k = int(rng.integers(1, n + 1))

        def before(a, b):
            return sel[a] > sel[b] or (sel[a] == sel[b] and a < b)

        ok = [set(s) for s in itertools.combinations(range(n), k)
              if all(before(a, b) for a in s for b in range(n) if b not in s)]
        assert len(ok) == 1
        assert set(H.select_topk(sel, k).tolist()) == ok[0]


# ---------------------------------------------------------------- selection-only path
def _tie_inputs(seed, B, Hq, Hkv, N, d, S):
    """Integer-valued queries, landmark keys and biases (d = 4: scale 1/2), so
    that scores are exact multiples of 1/2 and many of them tie exactly."""
    rng = np.random.default_rng(seed)
    C = N // S
    return dict(q=rng.integers(-1, 2, (B, Hq, N, d)).astype(float),
                k=rng.standard_normal((B, Hkv, N, d)), v=rng.standard_normal((B, Hkv, N, d)),
                kL=rng.integers(-1, 2, (B, Hkv, C, d)).astype(float),
                e=rng.integers(-1, 2, (B, Hkv, C)).astype(float))


def _brute_selection(t, b, g, i, S, W, scale):
    """Selection scores of row (b, g, i) from scalar loops only (Q-Cal
    included, per head or one shared pair)."""
    q = np.asarray(t["q"])
    Hq, Hkv = q.shape[1], t["k"].shape[1]
    G = Hq // Hkv
    qhat = []
    for hh in range(G):
        h = g * G + hh
        qv = q[b, h, i].tolist()
        if t.get("W_down") is not None:
            Wd = np.asarray(t["W_down"])
            Wu = np.asarray(t["W_up"])
            Wd, Wu = (Wd, Wu) if Wd.ndim == 2 else (Wd[h], Wu[h])
            qv = brute.qcal_row(qv, np.asarray(t["h"])[b, i].tolist(), Wd.tolist(), Wu.tolist())
        qhat.append(qv)
    nd = H.n_distant(i, W, S)
    _, sel = brute.selection_scores(qhat, np.asarray(t["kL"])[b, g].tolist(),
                                    np.asarray(t["e"])[b, g].tolist(), nd, scale)
    return sel


@pytest.mark.parametrize("case", ["ties_gqa2", "ties_mha", "qcal_gqa2", "qcal_shared_gqa4",
                                  "qcal_mha_bias"])
def test_route_matches_forward_and_scalar_rank_count(case):
    """hils_route (selection only) takes the same sets as hils_forward and as
    scalar scores ranked by the rank-count definition; its ranking is the
    rank-count order. Integer-valued cases tie exactly (a reversed tie-break
    fails them); the bias case shifts every bias by its chunk id (a bias
    taken from the wrong slice fails it)."""
    S, K, W, N = 4, 3, 6, 60
    if case.startswith("ties"):
        Hq, Hkv = (2, 1) if case == "ties_gqa2" else (1, 1)
        t = _tie_inputs(21 if Hq == 2 else 22, 2, Hq, Hkv, N, 4, S)
    else:
        Hq, Hkv = dict(qcal_gqa2=(2, 1), qcal_shared_gqa4=(4, 1), qcal_mha_bias=(2, 2))[case]
        t = small_inputs(23, B=2, Hq=Hq, Hkv=Hkv, N=N, d=8, S=S, qcal=True)
        if case == "qcal_shared_gqa4":
            t = _shared(t, 29)
        if case == "qcal_mha_bias":
            t["e"] = t["e"] + 0.25 * np.arange(N // S)[None, None, :]
    d = t["q"].shape[-1]
    sc = 1 / math.sqrt(d)
    rt = H.hils_route(t, S, K, W)
    fw = H.hils_forward(t, S, K, W)
    np.testing.assert_array_equal(rt["topk"], fw["topk"])
    ties = 0
    for b in range(2):
        for g in range(Hkv):
            for i in range(N):
                sel = _brute_selection(t, b, g, i, S, W, sc)
                nd = len(sel)
                ties += nd - len(set(sel))
                T = brute.rank_count_topk(sel, min(K, nd))
                got = [int(c) for c in rt["topk"][b, g, i] if c >= 0]
                assert got == T, (case, b, g, i, got, T)
                scores, order = rt["ranked"][(b, g, i)]
                assert list(order) == brute.rank_order(sel)
                np.testing.assert_allclose(scores, np.asarray(sel)[list(order)], rtol=0,
                                           atol=1e-12)
    if case.startswith("ties"):
        assert ties > 100  # the tie-break decides many rows


def test_decode_ranking_matches_scalar_rank_count():
    """The decode oracle's ranking of each (sequence, KV group) is the
    rank-count order of scalar scores at position seq_len - 1 (ragged
    lengths, GQA, Q-Cal per head and shared)."""
    S, K, W, N, d = 4, 3, 6, 52, 8
    for shared in (False, True):
        t = small_inputs(31, B=3, Hq=4, Hkv=2, N=N, d=d, S=S, qcal=True)
        if shared:
            t = _shared(t, 37)
        lens = [N, N - 7, 11]
        dec = dict(q=np.stack([t["q"][b, :, n - 1] for b, n in enumerate(lens)]), k=t["k"],
                   v=t["v"], kL=t["kL"], e=t["e"],
                   h=np.stack([t["h"][b, n - 1] for b, n in enumerate(lens)]),
                   W_down=t["W_down"], W_up=t["W_up"], seq_len=torch.tensor(lens))
        od = H.hils_decode(dec, S, K, W)
        ro = H.hils_decode(dict(dec, k=None, v=None), S, K, W, rank_only=True)
        np.testing.assert_array_equal(ro["topk"], od["topk"])
        for b, n in enumerate(lens):
            for g in range(2):
                np.testing.assert_array_equal(ro["ranked"][(b, g)][1], od["ranked"][(b, g)][1])
                sel = _brute_selection(t, b, g, n - 1, S, W, 1 / math.sqrt(d))
                scores, order = od["ranked"][(b, g)]
                assert list(order) == brute.rank_order(sel)
                np.testing.assert_allclose(scores, np.asarray(sel)[list(order)], rtol=0, atol=1e-12)
                T = brute.rank_count_topk(sel, min(K, len(sel)))
                assert [int(c) for c in od["topk"][b, g] if c >= 0] == T


# ---------------------------------------------------------------- window only
def test_no_distant_chunk_is_causal_window_attention():
    """Rows with no distant chunk reduce to textbook causal attention."""
    t = small_inputs(1, Hq=1, N=40, d=8, S=4, qcal=False)
    W = 64  # larger than N: no row has a distant chunk
    out = H.hils_forward(t, S=4, K=3, W=W)
    ref = full_causal_attention(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], 1 / math.sqrt(8))
    np.testing.assert_allclose(out["o"][0, 0], ref, atol=1e-12)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed,Hq,Hkv,qcal,shift", [(0, 2, 1, True, 0.0), (1, 1, 1, False, 3.0),
                                                    (2, 4, 2, True, 2.0)])
def test_vectorised_oracle_matches_brute_force(seed, Hq, Hkv, qcal, shift):
    S, K, W, N, d = 4, 3, 6, 56, 8
    t = small_inputs(seed, Hq=Hq, Hkv=Hkv, N=N, d=d, S=S, qcal=qcal, e_shift=shift)
    out = H.hils_forward(t, S, K, W, keep_rows=True)
    G = Hq // Hkv
    sc = 1 / math.sqrt(d)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        for i in range(N):
            r = out["rows"][(0, g, i)]
            T, o, L = brute.brute_row(t["q"][0, hs, i].tolist(), r.q_hat.tolist(),
                                      t["k"][0, g].tolist(), t["v"][0, g].tolist(),
                                      t["kL"][0, g].tolist(), t["e"][0, g].tolist(),
                                      i, S, K, W, sc)
            assert list(r.T) == T
            np.testing.assert_allclose(out["o"][0, hs, i], np.array(o), atol=1e-12)
            np.testing.assert_allclose(out["lse"][0, hs, i], np.array(L), atol=1e-12)


# ---------------------------------------------------------------- fusion invariants
def test_fusion_weights_sum_to_one_and_output_in_hull():
    t = small_inputs(5, Hq=2, N=80, d=8, S=4, e_shift=1.0)
    out = H.hils_forward(t, 4, 3, 6, keep_rows=True)
    V = t["v"][0, 0]
    for i in range(80):
        r = out["rows"][(0, 0, i)]
        w = np.exp(np.concatenate([r.s_T, r.l_W[:, None]], 1) - r.lse[:, None])
        np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-13)
        toks = [j for c in r.T for j in range(4 * c, 4 * c + 4)] + list(range(H.window_start(i, 6, 4), i + 1))
        lo, hi = V[toks].min(0), V[toks].max(0)
        assert np.all(r.o >= lo - 1e-12) and np.all(r.o <= hi + 1e-12)


def _all_distant_with_exact_scores(t, S, W, d):
    """Force T = every distant chunk and s_c = that chunk's exact log-sum-exp."""
    sc = 1 / math.sqrt(d)
    q = t["q"][0]
    N = q.shape[1]
    outs = []
    for i in range(N):
        nd = H.n_distant(i, W, S)
        T = list(range(nd))
        qr = q[:, i]
        s_T = np.array([[H.logsumexp(sc * qr[h] @ t["k"][0, 0, c * S:(c + 1) * S].T) for c in T]
                        for h in range(qr.shape[0])]).reshape(qr.shape[0], nd)
        r = H.row_forward(qr, qr, t["k"][0, 0], t["v"][0, 0], t["kL"][0, 0], t["e"][0, 0], i, S, 99,
                          W, sc, forced_T=T, forced_s_T=s_T)
        outs.append(r.o)
    return np.stack(outs, 1)


def test_all_chunks_with_exact_lse_equals_full_attention():
    """With every distant chunk selected and each surrogate replaced by the
    chunk's exact log-sum-exp, the output is full causal attention."""
    S, W, d, N = 4, 6, 8, 60
    t = small_inputs(6, Hq=1, N=N, d=d, S=S, qcal=False)
    o = _all_distant_with_exact_scores(t, S, W, d)
    ref = full_causal_attention(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], 1 / math.sqrt(d))
    np.testing.assert_allclose(o[0], ref, atol=1e-12)


def tangent_landmarks(q_row, K, S, C, scale):
    """Landmark key = softmax-weighted mean of the chunk's keys and bias =
    entropy of that softmax, both taken at the query q_row (the first-order
    Taylor expansion of the chunk's log-mass, paperglide 'The HiLS-Attention
    Mechanism', landmark-summary steps)."""
    kL = np.zeros((C, K.shape[1]))
    e = np.zeros(C)
    for c in range(C):
        x = scale * K[c * S:(c + 1) * S] @ q_row
        p = H.softmax(x)
        kL[c] = p @ K[c * S:(c + 1) * S]
        e[c] = -(p * np.log(p)).sum()
    return kL, e


def test_tangent_point_surrogate_equals_exact_chunk_lse_and_full_attention_grads():
    S, W, d, N = 4, 6, 8, 48
    sc = 1 / math.sqrt(d)
    t = small_inputs(7, Hq=1, N=N, d=d, S=S, qcal=False)
    i = N - 1
    q_row = t["q"][0, 0, i]
    kL, e = tangent_landmarks(q_row, t["k"][0, 0], S, N // S, sc)
    nd = H.n_distant(i, W, S)
    r = H.row_forward(q_row[None], q_row[None], t["k"][0, 0], t["v"][0, 0], kL, e, i, S, nd, W, sc)
    # s_c equals the exact chunk log-sum-exp for every distant chunk
    exact = np.array([H.logsumexp(sc * t["k"][0, 0, c * S:(c + 1) * S] @ q_row) for c in range(nd)])
    np.testing.assert_allclose(r.s[0], exact, atol=1e-12)
    # all chunks selected (K >= n_dist): output = full causal attention
    ref = full_causal_attention(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], sc)[i]
    np.testing.assert_allclose(r.o[0], ref, atol=1e-12)
    # gradients dq and dv equal those of full attention for loss dO . o_i
    dO = rnd(8, 1, d)
    dK = np.zeros_like(t["k"][0, 0]); dV = np.zeros_like(dK)
    dkL = np.zeros_like(kL); de = np.zeros_like(e)
    gr = H.row_backward(r, q_row[None], t["k"][0, 0], t["v"][0, 0], kL, i, S, W, sc, dO, dK, dV, dkL, de)
    Q = torch.tensor(q_row[None], requires_grad=True)
    Kt = torch.tensor(t["k"][0, 0, :i + 1], requires_grad=True)
    Vt = torch.tensor(t["v"][0, 0, :i + 1], requires_grad=True)
    a = torch.softmax(sc * Q @ Kt.T, -1)
    (a @ Vt * torch.tensor(dO)).sum().backward()
    np.testing.assert_allclose(gr.dq, Q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV[:i + 1], Vt.grad.numpy(), atol=1e-12)


def test_uniform_chunk_closed_form_and_gibbs_bound():
    """A chunk whose keys are all equal has log-mass scale*q.k + ln S, and the
    Taylor surrogate reproduces it exactly; for any other query the surrogate
    built at q' is a lower bound of the exact log-mass (Gibbs)."""
    S, d = 16, 8
    sc = 1 / math.sqrt(d)
    rng = np.random.default_rng(9)
    kap = rng.standard_normal(d)
    Kc = np.tile(kap, (S, 1))
    q = rng.standard_normal(d)
    kL, e = tangent_landmarks(rng.standard_normal(d), Kc, S, 1, sc)
    np.testing.assert_allclose(sc * q @ kL[0] + e[0], sc * q @ kap + math.log(S), atol=1e-12)
    np.testing.assert_allclose(H.logsumexp(sc * Kc @ q), sc * q @ kap + math.log(S), atol=1e-12)
    Kr = rng.standard_normal((S, d)) * 2
    qp = rng.standard_normal(d)
    kL, e = tangent_landmarks(qp, Kr, S, 1, sc)
    for _ in range(50):
        qq = rng.standard_normal(d) * 2
        assert sc * qq @ kL[0] + e[0] <= H.logsumexp(sc * Kr @ qq) + 1e-12
    np.testing.assert_allclose(sc * qp @ kL[0] + e[0], H.logsumexp(sc * Kr @ qp), atol=1e-12)


# ---------------------------------------------------------------- GQA
def test_gqa_group_of_one_is_per_head_selection_and_duplicate_heads_change_nothing():
    S, K, W, N, d = 4, 3, 6, 48, 8
    t = small_inputs(10, Hq=2, Hkv=2, N=N, d=d, S=S, qcal=False)
    out = H.hils_forward(t, S, K, W)
    for g in range(2):
        one = {kk: (vv[:, g:g + 1] if kk in ("q", "k", "v", "kL", "e") else vv) for kk, vv in t.items()}
        o1 = H.hils_forward(one, S, K, W)
        np.testing.assert_array_equal(o1["topk"][0, 0], out["topk"][0, g])
    # duplicate head 0 into a group of two sharing KV head 0: same selection
    t2 = dict(t)
    t2["q"] = np.concatenate([t["q"][:, :1], t["q"][:, :1]], 1)
    t2["k"], t2["v"], t2["kL"], t2["e"] = t["k"][:, :1], t["v"][:, :1], t["kL"][:, :1], t["e"][:, :1]
    o2 = H.hils_forward(t2, S, K, W)
    np.testing.assert_array_equal(o2["topk"][0, 0], out["topk"][0, 0])
    np.testing.assert_allclose(o2["o"][0, 1], out["o"][0, 0], atol=1e-13)


def test_gqa_selects_on_the_max_over_heads():
    """A chunk that only one head of the group likes is still selected."""
    S, K, W, N, d = 4, 1, 4, 40, 8
    t = small_inputs(11, Hq=2, Hkv=1, N=N, d=d, S=S, qcal=False)
    i = N - 1
    t["kL"][0, 0] = 0.0
    t["e"][0, 0] = 0.0
    t["kL"][0, 0, 2] = 20 * t["q"][0, 1, i]  # only head 1 scores chunk 2 highly
    out = H.hils_forward(t, S, K, W, rows=[i])
    assert out["topk"][0, 0, i, 0] == 2


# ---------------------------------------------------------------- needle (tiny workload)
def test_tiny_workload_needle():
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["tiny"]
    t = make_inputs(wl)
    i = wl.N - 1
    out = H.hils_forward(t, wl.S, wl.K, wl.W, rows=[i], keep_rows=True)
    r = out["rows"][(0, 0, i)]
    assert 7 in r.T
    q = H.f64(t["q"])[0, 0, i]
    v = H.f64(t["v"])[0, 0]
    t7 = list(r.T).index(7)
    # identical keys: the chunk's softmax is uniform and its log-mass closed-form
    np.testing.assert_allclose(r.O_c[0, t7], v[7 * 64:8 * 64].mean(0), atol=1e-12)
    kk = H.f64(t["k"])[0, 0, 7 * 64]
    np.testing.assert_allclose(r.l_c[0, t7], (q @ kk) / 8 + math.log(64), atol=1e-12)
    np.testing.assert_allclose((q @ kk) / 8, 3 * np.linalg.norm(q), rtol=1e-6)
    # its score is far above every other chunk's
    others = np.delete(r.sel, 7)
    assert r.sel[7] > others.max() + 3


# ---------------------------------------------------------------- backward
def _loss(t, dO, S, K, W, T):
    out = H.hils_forward(t, S, K, W, forced_topk=T)
    return float((out["o"] * dO).sum())


@pytest.mark.parametrize("seed,Hq,Hkv", [(12, 2, 1), (13, 2, 2)])
def test_backward_matches_finite_differences(seed, Hq, Hkv):
    S, K, W, N, d = 4, 3, 8, 44, 8
    t = small_inputs(seed, Hq=Hq, Hkv=Hkv, N=N, d=d, S=S, qcal=True, e_shift=1.5)
    dO = rnd(seed + 100, 1, Hq, N, d)
    g = H.hils_backward(t, dO, S, K, W)
    T = g["topk"]
    rng = np.random.default_rng(seed)
    eps = 1e-6
    names = dict(q="dq", k="dk", v="dv", kL="dkL", e="de", W_down="dW_down", W_up="dW_up", h="dh")
    for name, gname in names.items():
        for _ in range(2):
            u = rng.standard_normal(t[name].shape)
            tp = dict(t); tp[name] = t[name] + eps * u
            tm = dict(t); tm[name] = t[name] - eps * u
            fd = (_loss(tp, dO, S, K, W, T) - _loss(tm, dO, S, K, W, T)) / (2 * eps)
            an = float((g[gname] * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_fusion_score_gradients_sum_to_zero():
    """Shifting every fusion term by the same constant leaves the output
    unchanged, so the score gradients plus the window term's sum to zero."""
    S, K, W, N, d = 4, 3, 6, 40, 8
    t = small_inputs(14, Hq=2, N=N, d=d, S=S, e_shift=2.0)
    out = H.hils_forward(t, S, K, W, keep_rows=True)
    dO = rnd(15, 2, d)
    for i in range(N):
        r = out["rows"][(0, 0, i)]
        z = np.zeros_like(t["k"][0, 0])
        gr = H.row_backward(r, t["q"][0, :, i], t["k"][0, 0], t["v"][0, 0], t["kL"][0, 0], i, S, W,
                            1 / math.sqrt(d), dO, z.copy(), z.copy(), np.zeros_like(t["kL"][0, 0]),
                            np.zeros_like(t["e"][0, 0]))
        np.testing.assert_allclose(gr.ds.sum(1) + gr.dlW, 0.0, atol=1e-12)


# ---------------------------------------------------------------- decode
def test_decode_equals_last_prefill_row():
    S, K, W, N, d = 4, 3, 6, 52, 8
    t = small_inputs(16, B=2, Hq=4, Hkv=2, N=N, d=d, S=S, qcal=True)
    lens = [N, N - 5]
    dec = dict(q=np.stack([t["q"][b, :, n - 1] for b, n in enumerate(lens)]), k=t["k"], v=t["v"],
               kL=t["kL"], e=t["e"], h=np.stack([t["h"][b, n - 1] for b, n in enumerate(lens)]),
               W_down=t["W_down"], W_up=t["W_up"], seq_len=torch.tensor(lens))
    od = H.hils_decode(dec, S, K, W)
    for b, n in enumerate(lens):
        tb = {kk: (vv[b:b + 1, :, :n] if kk in ("q", "k", "v", "kL", "e") else
                   vv[b:b + 1, :n] if kk == "h" else vv) for kk, vv in t.items()}
        tb["kL"], tb["e"] = t["kL"][b:b + 1, :, :n // S], t["e"][b:b + 1, :, :n // S]
        of = H.hils_forward(tb, S, K, W, rows=[n - 1])
        np.testing.assert_allclose(od["o"][b], of["o"][0, :, n - 1], atol=1e-13)
        np.testing.assert_array_equal(od["topk"][b], of["topk"][0, :, n - 1])


# ---------------------------------------------------------------- landmark summary
def test_landmark_summary_taylor_point_and_gibbs_bound():
    """At its own landmark query the surrogate scale*q.kL + e equals the
    chunk's exact log-mass (scipy's logsumexp), and for any other query it
    lies below it (Gibbs); pins kL = sum p k and e = H(p) together."""
    from scipy.special import logsumexp as lse_ref
    S, d, C = 8, 8, 3
    sc = 1 / math.sqrt(d)
    rng = np.random.default_rng(41)
    qL = rng.standard_normal((1, 2, C, d)) * 1.5
    k = rng.standard_normal((1, 2, C * S + 5, d))
    kL, e = H.landmark_summary(qL, k, S)
    for g in range(2):
        for c in range(C):
            Kc = k[0, g, c * S:(c + 1) * S]
            exact = lse_ref(sc * Kc @ qL[0, g, c])
            assert abs(sc * qL[0, g, c] @ kL[0, g, c] + e[0, g, c] - exact) < 1e-12
            for _ in range(20):
                qq = rng.standard_normal(d) * 2
                assert sc * qq @ kL[0, g, c] + e[0, g, c] <= lse_ref(sc * Kc @ qq) + 1e-12


def test_landmark_summary_uniform_chunk_and_one_hot_limit():
    """All keys equal: the summary key is that key and the bias is ln S
    (uniform weights). A landmark query far along one key (orthogonal keys):
    the weights become one-hot, the summary key that key, the bias 0."""
    S, d = 16, 16
    rng = np.random.default_rng(42)
    kap = rng.standard_normal(d)
    k = np.tile(kap, (1, 1, S, 1))
    kL, e = H.landmark_summary(rng.standard_normal((1, 1, 1, d)), k, S)
    np.testing.assert_allclose(kL[0, 0, 0], kap, atol=1e-12)
    assert abs(e[0, 0, 0] - math.log(S)) < 1e-12
    eye = np.eye(S)[None, None]  # keys = unit vectors
    j = 5
    qL = (200.0 * eye[0, 0, j])[None, None, None]
    kL, e = H.landmark_summary(qL, eye, S)
    np.testing.assert_allclose(kL[0, 0, 0], eye[0, 0, j], atol=1e-10)
    assert 0.0 <= e[0, 0, 0] < 1e-10


def test_landmark_summary_two_token_example_structure():
    """The pages' two-token example: scores (0.2, 0.8) give the softmax
    weights, the weighted key and their entropy (scipy's softmax and
    entropy); the page's printed numbers are inconsistent with each other,
    so only the structure is checked."""
    from scipy.special import softmax as sm
    from scipy.stats import entropy
    d = 4
    sc = 1 / math.sqrt(d)
    k = np.array([[0.2, 1.0, -1.0, 0.5], [0.8, -0.3, 2.0, 0.0]])[None, None]
    qL = np.array([1.0 / sc, 0.0, 0.0, 0.0])[None, None, None]
    kL, e = H.landmark_summary(qL, k, 2)
    p = sm([0.2, 0.8])
    np.testing.assert_allclose(kL[0, 0, 0], p[0] * k[0, 0, 0] + p[1] * k[0, 0, 1], atol=1e-14)
    assert abs(e[0, 0, 0] - entropy(p)) < 1e-14
    np.testing.assert_allclose(p, [0.35434369, 0.64565631], atol=1e-8)


def test_landmark_backward_matches_autograd_and_finite_differences():
    """dqL and dk of E = sum dkL . kL + sum de e: torch fp64 autograd of the
    definition, and central differences of the oracle's forward."""
    S, d, C, N = 8, 8, 3, 29
    rng = np.random.default_rng(43)
    qL = rng.standard_normal((1, 2, C, d))
    k = rng.standard_normal((1, 2, N, d))
    dkL = rng.standard_normal((1, 2, C, d))
    de = rng.standard_normal((1, 2, C))
    dqL, dk = H.landmark_backward(qL, k, dkL, de, S)
    Q = torch.tensor(qL, requires_grad=True)
    Kt = torch.tensor(k, requires_grad=True)
    sc = 1 / math.sqrt(d)
    Kc = Kt[:, :, :C * S].reshape(1, 2, C, S, d)
    s = sc * torch.einsum("bgcsd,bgcd->bgcs", Kc, Q)
    logp = torch.log_softmax(s, -1)
    p = logp.exp()
    kLt = torch.einsum("bgcs,bgcsd->bgcd", p, Kc)
    et = -(p * logp).sum(-1)
    ((kLt * torch.tensor(dkL)).sum() + (et * torch.tensor(de)).sum()).backward()
    np.testing.assert_allclose(dqL, Q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, Kt.grad.numpy(), atol=1e-12)

    def E(qq, kk):
        a, b = H.landmark_summary(qq, kk, S)
        return (a * dkL).sum() + (b * de).sum()
    h = 1e-6
    for idx in [(0, 0, 1, 3), (0, 1, 2, 7)]:
        qp = qL.copy(); qp[idx] += h
        qm = qL.copy(); qm[idx] -= h
        assert abs((E(qp, k) - E(qm, k)) / (2 * h) - dqL[idx]) < 1e-7
    for idx in [(0, 0, 5, 2), (0, 1, 17, 0), (0, 1, 27, 4)]:
        kp = k.copy(); kp[idx] += h
        km = k.copy(); km[idx] -= h
        assert abs((E(qL, kp) - E(qL, km)) / (2 * h) - dk[idx]) < 1e-7


# ---------------------------------------------------------------- HoPE
def _hope_generator(d, thetas, pairs):
    """Skew-symmetric generator whose exponential turns each listed pair
    (a, b) by theta * position (counter-clockwise: a towards b)."""
    A = np.zeros((d, d))
    for (a, b), t in zip(pairs, thetas):
        A[b, a] = t
        A[a, b] = -t
    return A


@pytest.mark.parametrize("interleaved", [False, True])
def test_hope_is_the_exponential_of_its_rotation_generator(interleaved):
    """d = 8, base 1e4: theta = 1, 0.1, 0.01, 0.001 (10^-j), periods 6.28,
    62.8, 628, 6283. With a training length of 100 the first two pairs rotate
    and the last two carry no position. Every row must equal expm(pos A) x,
    with A built from the hand-written pairs, not from the oracle's tables."""
    from scipy.linalg import expm
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 5, 8))
    pos = rng.integers(0, 5000, size=(2, 5))
    pairs = [(0, 1), (2, 3), (4, 5), (6, 7)] if interleaved else [(0, 4), (1, 5), (2, 6), (3, 7)]
    A = _hope_generator(8, [1.0, 0.1, 0.0, 0.0], pairs)
    y = H.hope_rotate(x, pos, base=1e4, train_len=100, interleaved=interleaved)
    for b in range(2):
        for n in range(5):
            R = expm(pos[b, n] * A)
            for h in range(3):
                np.testing.assert_allclose(y[b, h, n], R @ x[b, h, n], rtol=0, atol=1e-9)
    yi = H.hope_rotate(x, pos, base=1e4, train_len=100, interleaved=interleaved, inverse=True)
    for b in range(2):
        for n in range(5):
            R = expm(-pos[b, n] * A)
            np.testing.assert_allclose(yi[b, 0, n], R @ x[b, 0, n], rtol=0, atol=1e-9)


def test_hope_period_cut_worked_numbers():
    """d = 64, base 1e4: pair j has period 2 pi 10^(j/8): pair 22 3533.3,
    pair 23 4711.7, pair 24 6283.19, pair 25 8378.8, pair 31 47117. A
    training length of 8192 keeps pairs 0 .. 24; 6283 keeps 0 .. 23; 6284
    keeps 0 .. 24 again; 4096 keeps 0 .. 22."""
    assert list(H.hope_rotating(64, 1e4, 8192)) == [True] * 25 + [False] * 7
    assert list(H.hope_rotating(64, 1e4, 6283)) == [True] * 24 + [False] * 8
    assert list(H.hope_rotating(64, 1e4, 6284)) == [True] * 25 + [False] * 7
    assert list(H.hope_rotating(64, 1e4, 4096)) == [True] * 23 + [False] * 9
    assert not H.hope_rotating(64, 1e4, 6).any()        # shortest period 2 pi
    assert H.hope_rotating(64, 1e4, 47118).all()       # longest 2 pi 10^(31/8)


def test_hope_worked_rotation_of_a_unit_vector():
    """One pair, theta_0 = 1: the unit vector (1, 0) at position p becomes
    (cos p, sin p); at position 1: (0.5403023058681398, 0.8414709848078965)."""
    x = np.zeros((1, 1, 3, 2))
    x[..., 0] = 1.0
    y = H.hope_rotate(x, None, base=1e4, train_len=10)
    np.testing.assert_allclose(y[0, 0, 0], [1.0, 0.0], atol=1e-15)
    np.testing.assert_allclose(y[0, 0, 1], [0.5403023058681398, 0.8414709848078965], atol=1e-15)
    np.testing.assert_allclose(y[0, 0, 2], [-0.4161468365471424, 0.9092974268256817], atol=1e-15)


def test_hope_scores_depend_on_relative_position_only_and_nope_part_on_none():
    """<R(m) q, R(n) k> is unchanged when both positions shift by the same
    amount (rotations compose); the NoPE pairs contribute the plain product
    whatever the positions; nothing rotates below the shortest period."""
    rng = np.random.default_rng(3)
    d = 16
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    rot = H.hope_rotating(d, 1e4, 200)
    assert rot.any() and not rot.all()
    a, b = H.hope_pairs(d, False)
    nope = np.concatenate([a[~rot], b[~rot]])

    def score(m, n):
        return float((H.hope_rotate(q, [[m]], 1e4, 200) * H.hope_rotate(k, [[n]], 1e4, 200)).sum())

    for m, n in [(10, 3), (700, 650), (123456, 100000)]:
        for s in (1, 17, 4096):
            assert abs(score(m, n) - score(m + s, n + s)) < 1e-9
    # positions change the rotating part only
    qn = H.hope_rotate(q, [[999]], 1e4, 200)
    np.testing.assert_allclose(qn[..., nope], q[..., nope], rtol=0, atol=0)
    np.testing.assert_allclose(H.hope_rotate(q, [[999]], 1e4, 5), q, rtol=0, atol=0)


def test_hope_inverse_is_the_transpose_and_pairs_keep_their_norm():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 2, 7, 64))
    y = rng.standard_normal((2, 2, 7, 64))
    pos = rng.integers(0, 1 << 20, size=(2, 7))
    for il in (False, True):
        Rx = H.hope_rotate(x, pos, 1e4, 8192, interleaved=il)
        np.testing.assert_allclose(H.hope_rotate(Rx, pos, 1e4, 8192, interleaved=il, inverse=True), x,
                                   rtol=0, atol=1e-12)
        RTy = H.hope_rotate(y, pos, 1e4, 8192, interleaved=il, inverse=True)
        assert abs((Rx * y).sum() - (x * RTy).sum()) < 1e-9
        a, b = H.hope_pairs(64, il)
        np.testing.assert_allclose(Rx[..., a] ** 2 + Rx[..., b] ** 2, x[..., a] ** 2 + x[..., b] ** 2,
                                   rtol=1e-12)


def test_hope_interleaved_layout_is_a_permutation_of_the_split_layout():
    """Moving dims (j, j + d/2) to (2j, 2j + 1) maps one convention onto the
    other."""
    rng = np.random.default_rng(9)
    d = 64
    x = rng.standard_normal((1, 3, 11, d))
    pos = rng.integers(0, 100000, size=(1, 11))
    perm = np.empty(d, dtype=int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2      # interleaved slot -> split dim
    ys = H.hope_rotate(x, pos, 1e4, 8192)
    yi = H.hope_rotate(x[..., perm], pos, 1e4, 8192, interleaved=True)
    np.testing.assert_allclose(yi, ys[..., perm], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- shared Q-Cal
def _shared(t, seed):
    """The same inputs with one Q-Cal pair for all heads (W_down [r, D],
    W_up [d, r])."""
    rng = np.random.default_rng(seed)
    Hq, r, D = t["W_down"].shape
    d = t["W_up"].shape[1]
    ts = dict(t)
    ts["W_down"] = rng.standard_normal((r, D)) * 0.3
    ts["W_up"] = rng.standard_normal((d, r)) * 0.3
    return ts


def test_shared_qcal_is_the_per_head_form_with_equal_pairs():
    """Sharing one pair is the per-head form with that pair in every head:
    prefill outputs, selections, decode, and (gradients of a tied weight) the
    per-head gradients summed over heads."""
    S, K, W, N, d = 4, 3, 8, 44, 8
    t = _shared(small_inputs(3, Hq=4, Hkv=2, N=N, d=d, S=S, qcal=True, e_shift=1.5), 7)
    tp = dict(t)
    tp["W_down"] = np.repeat(t["W_down"][None], 4, axis=0)
    tp["W_up"] = np.repeat(t["W_up"][None], 4, axis=0)
    dO = rnd(5, 1, 4, N, d)
    a = H.hils_backward(t, dO, S, K, W)
    b = H.hils_backward(tp, dO, S, K, W)
    assert a["dW_down"].shape == t["W_down"].shape and a["dW_up"].shape == t["W_up"].shape
    np.testing.assert_array_equal(a["topk"], b["topk"])
    for n in ("o", "lse", "dq", "dk", "dv", "dkL", "de", "dh"):
        np.testing.assert_allclose(a[n], b[n], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["dW_down"], b["dW_down"].sum(0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["dW_up"], b["dW_up"].sum(0), rtol=0, atol=1e-12)
    td = dict(t, q=t["q"][:, :, -1], h=t["h"][:, -1], seq_len=torch.tensor([N]))
    tdp = dict(tp, q=t["q"][:, :, -1], h=t["h"][:, -1], seq_len=torch.tensor([N]))
    x, y = H.hils_decode(td, S, K, W), H.hils_decode(tdp, S, K, W)
    np.testing.assert_allclose(x["o"], y["o"], rtol=0, atol=1e-12)


def test_shared_qcal_backward_matches_finite_differences():
    """Gradients with a shared pair against central differences of the
    oracle's own forward (the tied weight moves in every head at once)."""
    S, K, W, N, d = 4, 3, 8, 44, 8
    t = _shared(small_inputs(11, Hq=4, Hkv=2, N=N, d=d, S=S, qcal=True, e_shift=1.5), 13)
    dO = rnd(111, 1, 4, N, d)
    g = H.hils_backward(t, dO, S, K, W)
    T = g["topk"]
    rng = np.random.default_rng(11)
    eps = 1e-6
    for name, gname in dict(W_down="dW_down", W_up="dW_up", h="dh", q="dq").items():
        for _ in range(2):
            u = rng.standard_normal(np.shape(t[name]))
            tp = dict(t); tp[name] = t[name] + eps * u
            tm = dict(t); tm[name] = t[name] - eps * u
            fd = (_loss(tp, dO, S, K, W, T) - _loss(tm, dO, S, K, W, T)) / (2 * eps)
            an = float((g[gname] * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
