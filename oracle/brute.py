"""Pure-Python per-token HiLS forward for tiny inputs (test infrastructure).

An independent second reading of the same method (see hils_oracle for the
page citations): scalar loops only, top-K by the rank-count definition, and
the fusion written in token form, i.e. token j of selected chunk c gets the
weight exp(x_j + s_c - lse_c - L) and window token j the weight exp(x_j - L),
with L = log(sum over selected c of exp(s_c) + sum over window j of exp(x_j)).
Only for inputs of a few hundred tokens.
"""
from __future__ import annotations

import math


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def rank_count_topk(sel, k):
    """c is selected iff fewer than k chunks beat it, where c' beats c when
    sel[c'] > sel[c], or sel[c'] == sel[c] and c' < c."""
    out = []
    for c in range(len(sel)):
        beats = sum(1 for c2 in range(len(sel))
                    if sel[c2] > sel[c] or (sel[c2] == sel[c] and c2 < c))
        if beats < k:
            out.append(c)
    return out


def qcal_row(q, hvec, W_down, W_up):
    """q_hat = q + W_up (W_down h) for one head, by scalar loops (W_down r x D,
    W_up d x r as nested lists)."""
    u = [dot(row, hvec) for row in W_down]
    return [q[t] + dot(W_up[t], u) for t in range(len(q))]


def selection_scores(qhat, kL, e, nd, scale):
    """Per-head surrogate scores s[h][c] and the group's selection score
    sel[c] = max over heads, by scalar loops over the nd distant chunks."""
    s = [[scale * dot(qh, kL[c]) + e[c] for c in range(nd)] for qh in qhat]
    sel = [max(s[h][c] for h in range(len(qhat))) for c in range(nd)]
    return s, sel


def rank_order(sel):
    """Chunk ids sorted so that c comes before c' when it beats c' (higher
    score, or equal score and lower id), by counting how many beat each."""
    n = len(sel)
    pos = [sum(1 for c2 in range(n) if sel[c2] > sel[c] or (sel[c2] == sel[c] and c2 < c))
           for c in range(n)]
    out = [0] * n
    for c, p in enumerate(pos):
        out[p] = c
    return out


def lse(xs):
    m = max(xs)
    return m + math.log(sum(math.exp(x - m) for x in xs))


def brute_row(q, qhat, K, V, kL, e, i, S, Ktop, W, scale):
    """q, qhat: lists of G vectors; K, V: lists of token vectors; kL: list of
    chunk vectors; e: list. Returns (T, o[G][d], L[G])."""
    G = len(q)
    d = len(q[0])
    nd = max(0, (i - W + 1) // S)
    s = [[scale * dot(qhat[h], kL[c]) + e[c] for c in range(nd)] for h in range(G)]
    sel = [max(s[h][c] for h in range(G)) for c in range(nd)]
    T = rank_count_topk(sel, min(Ktop, nd))
    o = []
    Ls = []
    for h in range(G):
        win = list(range(nd * S, i + 1))
        xw = [scale * dot(q[h], K[j]) for j in win]
        L = lse([s[h][c] for c in T] + xw)   # log(sum exp s_c + sum exp x_j)
        acc = [0.0] * d
        for c in T:
            toks = range(c * S, (c + 1) * S)
            xc = [scale * dot(q[h], K[j]) for j in toks]
            lc = lse(xc)
            for x, j in zip(xc, toks):
                wgt = math.exp(x + s[h][c] - lc - L)
                for t in range(d):
                    acc[t] += wgt * V[j][t]
        for x, j in zip(xw, win):
            wgt = math.exp(x - L)
            for t in range(d):
                acc[t] += wgt * V[j][t]
        o.append(acc)
        Ls.append(L)
    return T, o, Ls
