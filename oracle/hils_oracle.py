"""HiLS attention: plain fp64 CPU oracle (test infrastructure, not product code).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. It shares no code with the GPU library and does not
import it.

It follows the method as described in "Hierarchical Sparse Attention Done
Right: Toward Infinite Context Modeling" (Hu et al.; pages: the paperglide
reader, the engineersofai abstract, the dev.to and nestfrontier summaries),
step by step and row by row, in float64 NumPy:

  1. Q-Cal (paperglide, "Implementation and Training Recipes", the Q-Cal
     worked example; dev.to, "Engineering Details"): the scoring query is
     q_hat = q + W_up (W_down h); token-level attention keeps the raw q. The
     pair is per query head, or one pair shared by all heads (W_down [r, D],
     W_up [d, r]; its gradient is then the sum over the heads).
  2. Surrogate chunk score (paperglide, "The HiLS-Attention Mechanism", the
     worked surrogate-score step and Fig. 3): s_c = q_hat . kL_c / sqrt(d) + e_c
     for every distant chunk, i.e. a complete chunk whose newest token is at
     least W positions older than the query.
  3. GQA (paperglide, Q-Cal section, the paragraph on query heads sharing a
     KV head): each head scores the chunks, the group selects on the
     maximum over its heads.
  4. Top-K selection (paperglide, worked example "top-K = 2 chunks are
     kept"; nestfrontier, "The routing problem"): the K best distant chunks
     by score, ties going to the lower chunk index.
  5. Token-level softmax inside each selected chunk and inside the local
     sliding window (paperglide, "Limitations of Naive Sparse Attention" and
     the intra-chunk step; nestfrontier, "The routing problem").
  6. Hierarchical fusion (paperglide Fig. 3: inter-chunk softmax assigns each
     chunk its mass, the intra-chunk softmax spreads it over the tokens;
     engineersofai abstract: the per-chunk outputs are fused according to
     the retrieval scores): a softmax over {s_c of the selected chunks,
     log-sum-exp of the window} weights the per-chunk outputs and the
     window output.

Readings taken where the pages are silent (each is listed in the design
notes of the repository):
  * the window is every token after the last distant chunk, so it spans
    W .. W+S-1 tokens and starts on a chunk boundary; its chunk-level term in
    the fusion is its exact log-sum-exp;
  * only complete chunks carry a landmark;
  * the scale 1/sqrt(d) applies to both the surrogate and the token logits
    (paperglide Q-Cal example divides by sqrt(d); Fig. 3 omits it "for
    simplicity");
  * each head fuses with its own scores s_{h,c} over the group's shared set;
  * fewer than K distant chunks: all are taken; none: plain causal window
    attention.

Upstream of step 2, landmark_summary builds kL and e themselves from each
chunk's landmark query (paperglide, "The HiLS-Attention Mechanism", the
landmark worked example), with its chain-rule backward landmark_backward.

hope_rotate applies HoPE, the partial rotary position encoding of queries and
keys (paperglide, "Implementation and Training Recipes"; dev.to, "Engineering
Details"), ahead of all of the above. The paperglide page also describes HoPE
as additive embeddings at token and chunk granularity; that reading is not
the one built (the two other passages agree on partial rotation).

The backward pass is not printed on the pages; it is the chain rule applied
to steps 1-6 with the selected set held fixed (selection is not
differentiated), and is pinned by finite differences in the tests.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def per_head(W, Hq: int):
    """Q-Cal factors as one matrix per query head: [Hq, a, b] as given, or a
    single shared [a, b] (one pair for all heads) repeated Hq times."""
    if W is None:
        return None
    W = f64(W)
    return np.repeat(W[None], Hq, axis=0) if W.ndim == 2 else W


def f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (any dtype) or array to float64 NumPy."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def n_distant(i: int, W: int, S: int) -> int:
    """Number of distant chunks for the query at position i: chunks c with
    newest token c*S + S - 1 <= i - W."""
    return max(0, (i - W + 1) // S)


def window_start(i: int, W: int, S: int) -> int:
    return n_distant(i, W, S) * S


def logsumexp(x: np.ndarray, axis=-1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))).squeeze(axis)


def softmax(x: np.ndarray, axis=-1) -> np.ndarray:
    return np.exp(x - np.expand_dims(logsumexp(x, axis), axis))


def rank_chunks(sel: np.ndarray) -> np.ndarray:
    """Chunk ids ordered by (selection score desc, chunk id asc): the order in
    which top-K takes them (ties go to the lower chunk index)."""
    return np.lexsort((np.arange(sel.shape[0]), -sel))


def select_topk(sel: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best entries of `sel` ordered by (score desc, index
    asc), returned in ascending index order."""
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rank_chunks(sel)[:k])


def surrogate_scores(q_hat: np.ndarray, kL: np.ndarray, e: np.ndarray, nd: int, scale: float):
    """Step 2 and the GQA max of step 3 for one query position of one KV group.

    q_hat: [G, d]; kL: [>= nd, d]; e: [>= nd]. Returns s [G, nd] with
    s[h, c] = scale * q_hat_h . kL_c + e_c over the nd distant chunks, and the
    group's selection score sel [nd] = the max of s over the heads."""
    s = scale * (q_hat @ kL[:nd].T) + e[None, :nd]
    sel = s.max(axis=0) if nd > 0 else np.zeros(0)
    return s, sel


def qcal(q: np.ndarray, hvec: Optional[np.ndarray], W_down: Optional[np.ndarray],
         W_up: Optional[np.ndarray]):
    """Calibrated scoring query for each head of one token.

    q: [G, d]; hvec: [D]; W_down: [G, r, D]; W_up: [G, d, r].
    Returns (q_hat [G, d], u [G, r] or None)."""
    if W_down is None or W_down.shape[1] == 0:
        return q.copy(), None
    u = np.einsum("grD,D->gr", W_down, hvec)
    dq = np.einsum("gdr,gr->gd", W_up, u)
    return q + dq, u


# --------------------------------------------------------------------------
# one query position of one KV group
# --------------------------------------------------------------------------
@dataclass
class RowResult:
    T: np.ndarray           # selected chunk ids, ascending
    s: np.ndarray           # [G, nd] surrogate scores of all distant chunks
    sel: np.ndarray         # [nd] group selection score (max over heads)
    o: np.ndarray           # [G, d]
    lse: np.ndarray         # [G] fusion log-normaliser L
    l_W: np.ndarray         # [G] window log-sum-exp
    O_W: np.ndarray         # [G, d] window output (normalised)
    l_c: np.ndarray         # [G, |T|] per-chunk log-sum-exp
    O_c: np.ndarray         # [G, |T|, d] per-chunk outputs (normalised)
    s_T: np.ndarray         # [G, |T|] scores used in the fusion
    q_hat: np.ndarray       # [G, d]
    u: Optional[np.ndarray]  # [G, r]


def row_forward(q: np.ndarray, q_hat: np.ndarray, K: np.ndarray, V: np.ndarray,
                kL: np.ndarray, e: np.ndarray, i: int, S: int, Ktop: int, W: int,
                scale: float, forced_T: Optional[Sequence[int]] = None,
                forced_s_T: Optional[np.ndarray] = None, u=None) -> RowResult:
    """HiLS forward for query position i of one KV group.

    q, q_hat: [G, d]; K, V: [>= i+1, d] keys/values of the group; kL: [C, d];
    e: [C]. forced_T replaces the selection; forced_s_T ([G, |T|]) replaces
    the fusion scores of the selected chunks."""
    nd = n_distant(i, W, S)
    # step 2/3: surrogate scores of every distant chunk, per head, and the
    # group's selection score (max over its heads)
    s, sel = surrogate_scores(q_hat, kL, e, nd, scale)
    # step 4: top-K
    if forced_T is None:
        T = select_topk(sel, min(Ktop, nd))
    else:
        T = np.asarray(sorted(int(c) for c in forced_T if c >= 0), dtype=np.int64)
    s_T = s[:, T] if forced_s_T is None else np.asarray(forced_s_T, dtype=np.float64)
    # step 5a: window [nd*S, i] (causal), exact softmax
    ws = nd * S
    xw = scale * (q @ K[ws:i + 1].T)               # [G, i+1-ws]
    l_W = logsumexp(xw)
    O_W = softmax(xw) @ V[ws:i + 1]
    # step 5b: each selected chunk, exact softmax over its S tokens
    G, d = q.shape
    l_c = np.zeros((G, len(T)))
    O_c = np.zeros((G, len(T), d))
    for t, c in enumerate(T):
        xc = scale * (q @ K[c * S:(c + 1) * S].T)  # [G, S]
        l_c[:, t] = logsumexp(xc)
        O_c[:, t] = softmax(xc) @ V[c * S:(c + 1) * S]
    # step 6: fusion softmax over {s_c, c in T} and the window's log-sum-exp
    terms = np.concatenate([s_T, l_W[:, None]], axis=1)  # [G, |T|+1]
    L = logsumexp(terms)
    w = np.exp(terms - L[:, None])
    o = np.einsum("gt,gtd->gd", w[:, :-1], O_c) + w[:, -1:] * O_W
    return RowResult(T=T, s=s, sel=sel, o=o, lse=L, l_W=l_W, O_W=O_W, l_c=l_c, O_c=O_c,
                     s_T=s_T, q_hat=q_hat, u=u)


@dataclass
class RowGrads:
    dq: np.ndarray        # [G, d] (token path + surrogate path)
    dq_hat: np.ndarray    # [G, d] surrogate path only
    ds: np.ndarray        # [G, |T|] gradient of each selected fusion score
    dlW: np.ndarray       # [G] gradient of the window's log-sum-exp term


def row_backward(r: RowResult, q: np.ndarray, K: np.ndarray, V: np.ndarray, kL: np.ndarray,
                 i: int, S: int, W: int, scale: float, dO: np.ndarray,
                 dK: np.ndarray, dV: np.ndarray, dkL: np.ndarray, de: np.ndarray) -> RowGrads:
    """Chain rule through row_forward with the selection held fixed.

    Accumulates into dK, dV ([N, d]), dkL ([C, d]) and de ([C]); returns the
    per-row query gradients."""
    G, d = q.shape
    T = r.T
    nd = n_distant(i, W, S)
    ws = nd * S
    D = np.einsum("gd,gd->g", dO, r.o)                       # dO . O
    w_c = np.exp(r.s_T - r.lse[:, None])                       # fusion weights
    w_W = np.exp(r.l_W - r.lse)
    delta_c = np.einsum("gd,gtd->gt", dO, r.O_c)               # dO . O_c
    delta_W = np.einsum("gd,gd->g", dO, r.O_W)
    ds = w_c * (delta_c - D[:, None])                           # d loss / d s_c
    dlW = w_W * (delta_W - D)
    dq = np.zeros((G, d))
    # window tokens: a_j = exp(x_j - L); dx_j = a_j (dO.v_j - D)
    xw = scale * (q @ K[ws:i + 1].T)
    a = np.exp(xw - r.lse[:, None])
    dp = dO @ V[ws:i + 1].T
    dx = a * (dp - D[:, None])
    dq += scale * dx @ K[ws:i + 1]
    dK[ws:i + 1] += scale * dx.T @ q
    dV[ws:i + 1] += a.T @ dO
    # selected chunk tokens: a_j = w_c p_j; dx_j = a_j (dO.v_j - delta_c)
    for t, c in enumerate(T):
        sl = slice(c * S, (c + 1) * S)
        xc = scale * (q @ K[sl].T)
        p = np.exp(xc - r.l_c[:, t:t + 1])
        a = w_c[:, t:t + 1] * p
        dp = dO @ V[sl].T
        dx = a * (dp - delta_c[:, t:t + 1])
        dq += scale * dx @ K[sl]
        dK[sl] += scale * dx.T @ q
        dV[sl] += a.T @ dO
    # surrogate path: s_c = scale q_hat . kL_c + e_c
    dq_hat = scale * ds @ kL[T] if len(T) else np.zeros((G, d))
    if len(T):
        dkL[T] += scale * ds.T @ r.q_hat
        de[T] += ds.sum(axis=0)
    return RowGrads(dq=dq + dq_hat, dq_hat=dq_hat, ds=ds, dlW=dlW)


# --------------------------------------------------------------------------
# whole-tensor drivers
# --------------------------------------------------------------------------
def _scale(d, scale):
    return 1.0 / math.sqrt(d) if not scale else float(scale)


class Problem:
    """fp64 copies of one call's inputs (prefill layout, see workloads)."""

    def __init__(self, t: dict, S: int, K: int, W: int, scale: Optional[float] = None):
        self.q = f64(t["q"])
        self.k = f64(t["k"])
        self.v = f64(t["v"])
        self.kL = f64(t["kL"])
        self.e = f64(t["e"])
        self.h = f64(t["h"]) if t.get("h") is not None else None
        self.B, self.Hq = self.q.shape[0], self.q.shape[1]
        # a shared Q-Cal pair ([r, D], [d, r]) is the same matrix for every head
        self.qcal_shared = t.get("W_down") is not None and f64(t["W_down"]).ndim == 2
        self.W_down = per_head(t.get("W_down"), self.Hq)
        self.W_up = per_head(t.get("W_up"), self.Hq)
        self.S, self.K, self.W = S, K, W
        self.Hkv = self.k.shape[1]
        self.G = self.Hq // self.Hkv
        self.d = self.q.shape[-1]
        self.scale = _scale(self.d, scale)

    def heads(self, g):
        return slice(g * self.G, (g + 1) * self.G)

    def qhat_row(self, b, g, i, q_row):
        if self.W_down is None:
            return q_row.copy(), None
        hs = self.heads(g)
        return qcal(q_row, self.h[b, i], self.W_down[hs], self.W_up[hs])


def hils_forward(t: dict, S: int, K: int, W: int, scale: Optional[float] = None,
                 rows: Optional[Sequence[int]] = None, batches: Optional[Sequence[int]] = None,
                 groups: Optional[Sequence[int]] = None, forced_topk=None, keep_rows=False):
    """Prefill forward. Returns dict with o [B,Hq,N,d], lse [B,Hq,N],
    topk [B,Hkv,N,K] (ascending, -1 padded). When rows/batches/groups are
    given only those (b, g, i) are computed (others stay NaN / -2)."""
    P = Problem(t, S, K, W, scale)
    B, Hq, N, d = P.q.shape
    o = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    topk = np.full((B, P.Hkv, N, K), -2, dtype=np.int64)
    rowres = {}
    forced = None if forced_topk is None else np.asarray(forced_topk)
    for b in (range(B) if batches is None else batches):
        for g in (range(P.Hkv) if groups is None else groups):
            hs = P.heads(g)
            for i in (range(N) if rows is None else rows):
                q_row = P.q[b, hs, i]
                q_hat, u = P.qhat_row(b, g, i, q_row)
                fT = None if forced is None else forced[b, g, i]
                r = row_forward(q_row, q_hat, P.k[b, g], P.v[b, g], P.kL[b, g], P.e[b, g], i,
                                S, K, W, P.scale, forced_T=fT, u=u)
                o[b, hs, i] = r.o
                lse[b, hs, i] = r.lse
                topk[b, g, i] = -1
                topk[b, g, i, :len(r.T)] = r.T
                if keep_rows:
                    rowres[(b, g, i)] = r
    out = dict(o=o, lse=lse, topk=topk)
    if keep_rows:
        out["rows"] = rowres
    return out


def hils_backward(t: dict, dO, S: int, K: int, W: int, scale: Optional[float] = None,
                  forced_topk=None, batches: Optional[Sequence[int]] = None,
                  groups: Optional[Sequence[int]] = None):
    """Training backward (whole sequences of the chosen batches / groups).

    Returns fp64 gradients dq, dk, dv, dkL, de, dW_down, dW_up, dh (Q-Cal ones
    only when Q-Cal is on), plus the forward outputs it recomputed."""
    P = Problem(t, S, K, W, scale)
    dO = f64(dO)
    B, Hq, N, d = P.q.shape
    C = P.kL.shape[2]
    dq = np.zeros_like(P.q)
    dk = np.zeros_like(P.k)
    dv = np.zeros_like(P.v)
    dkL = np.zeros_like(P.kL)
    de = np.zeros_like(P.e)
    qc = P.W_down is not None
    dWd = np.zeros_like(P.W_down) if qc else None
    dWu = np.zeros_like(P.W_up) if qc else None
    dh = np.zeros_like(P.h) if qc else None
    o = np.full((B, Hq, N, d), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    topk = np.full((B, P.Hkv, N, K), -2, dtype=np.int64)
    forced = None if forced_topk is None else np.asarray(forced_topk)
    for b in (range(B) if batches is None else batches):
        for g in (range(P.Hkv) if groups is None else groups):
            hs = P.heads(g)
            for i in range(N):
                q_row = P.q[b, hs, i]
                q_hat, u = P.qhat_row(b, g, i, q_row)
                fT = None if forced is None else forced[b, g, i]
                r = row_forward(q_row, q_hat, P.k[b, g], P.v[b, g], P.kL[b, g], P.e[b, g], i,
                                S, K, W, P.scale, forced_T=fT, u=u)
                o[b, hs, i] = r.o
                lse[b, hs, i] = r.lse
                topk[b, g, i] = -1
                topk[b, g, i, :len(r.T)] = r.T
                gr = row_backward(r, q_row, P.k[b, g], P.v[b, g], P.kL[b, g], i, S, W, P.scale,
                                  dO[b, hs, i], dk[b, g], dv[b, g], dkL[b, g], de[b, g])
                dq[b, hs, i] = gr.dq
                if qc:
                    # q_hat = q + W_up u, u = W_down h: back through the low-rank map
                    ddq = gr.dq_hat                                   # [G, d]
                    dWu[hs] += np.einsum("gd,gr->gdr", ddq, u)
                    du = np.einsum("gdr,gd->gr", P.W_up[hs], ddq)
                    dWd[hs] += np.einsum("gr,D->grD", du, P.h[b, i])
                    dh[b, i] += np.einsum("grD,gr->D", P.W_down[hs], du)
    if qc and P.qcal_shared:
        # one pair used by every head: its gradient sums the heads' uses
        dWd, dWu = dWd.sum(axis=0), dWu.sum(axis=0)
    return dict(dq=dq, dk=dk, dv=dv, dkL=dkL, de=de, dW_down=dWd, dW_up=dWu, dh=dh,
                o=o, lse=lse, topk=topk)


def hils_decode(t: dict, S: int, K: int, W: int, scale: Optional[float] = None,
                batches: Optional[Sequence[int]] = None, groups: Optional[Sequence[int]] = None,
                forced_topk=None, rank_only: bool = False):
    """Single-query decode: the new token sits at position seq_len[b]-1 and
    its key/value are already in the cache. q: [B,Hq,d]; k/v cache
    [B,Hkv,Nmax,d]; h: [B,D]. Returns o [B,Hq,d], lse [B,Hq], topk [B,Hkv,K]
    and ranked[(b, g)] = (selection scores in rank order, chunk ids in rank
    order) over the distant chunks of that sequence and KV group, for the
    near-tie checks of a selection computed elsewhere. With rank_only, only
    steps 1-4 run (topk and ranked; the caches are not read)."""
    q = f64(t["q"])
    B, Hq, d = q.shape
    Hkv = t["kL"].shape[1]
    G = Hq // Hkv
    sc = _scale(d, scale)
    seq = [int(x) for x in (t["seq_len"].tolist() if t.get("seq_len") is not None
                            else [t["k"].shape[2]] * B)]
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    topk = np.full((B, Hkv, K), -2, dtype=np.int64)
    ranked = {}
    qc = t.get("W_down") is not None
    Wd, Wu = per_head(t.get("W_down"), Hq), per_head(t.get("W_up"), Hq)
    for b in (range(B) if batches is None else batches):
        n = seq[b]
        i = n - 1
        for g in (range(Hkv) if groups is None else groups):
            hs = slice(g * G, (g + 1) * G)
            C = n // S
            kL = f64(t["kL"][b, g, :C])
            e = f64(t["e"][b, g, :C])
            if qc:
                q_hat, u = qcal(q[b, hs], f64(t["h"][b]), Wd[hs], Wu[hs])
            else:
                q_hat, u = q[b, hs].copy(), None
            if rank_only:
                nd = n_distant(i, W, S)
                _, sel = surrogate_scores(q_hat, kL, e, nd, sc)
                order = rank_chunks(sel)
                T = np.sort(order[:min(K, nd)])
                topk[b, g] = -1
                topk[b, g, :len(T)] = T
                ranked[(b, g)] = (sel[order], order)
                continue
            Kc = f64(t["k"][b, g, :n])
            Vc = f64(t["v"][b, g, :n])
            fT = None if forced_topk is None else np.asarray(forced_topk)[b, g]
            r = row_forward(q[b, hs], q_hat, Kc, Vc, kL, e, i, S, K, W, sc, forced_T=fT, u=u)
            o[b, hs] = r.o
            lse[b, hs] = r.lse
            topk[b, g] = -1
            topk[b, g, :len(r.T)] = r.T
            order = rank_chunks(r.sel)
            ranked[(b, g)] = (r.sel[order], order)
    return dict(o=o, lse=lse, topk=topk, ranked=ranked)


def hils_route(t: dict, S: int, K: int, W: int, scale: Optional[float] = None,
               rows: Optional[Sequence[int]] = None, batches=None, groups=None):
    """Selection only: topk [B,Hkv,N,K] and the sorted selection scores of
    every row (for near-tie checks): sel_sorted[(b,g,i)] = scores in
    (score desc, index asc) order."""
    P = Problem(t, S, K, W, scale)
    B, Hq, N, d = P.q.shape
    topk = np.full((B, P.Hkv, N, K), -2, dtype=np.int64)
    ranked = {}
    for b in (range(B) if batches is None else batches):
        for g in (range(P.Hkv) if groups is None else groups):
            hs = P.heads(g)
            for i in (range(N) if rows is None else rows):
                q_hat, _ = P.qhat_row(b, g, i, P.q[b, hs, i])
                nd = n_distant(i, W, S)
                # the same steps 1-4 as row_forward, without the attention
                _, sel = surrogate_scores(q_hat, P.kL[b, g], P.e[b, g], nd, P.scale)
                order = rank_chunks(sel)
                T = np.sort(order[:min(K, nd)])
                topk[b, g, i] = -1
                topk[b, g, i, :len(T)] = T
                ranked[(b, g, i)] = (sel[order], order)
    return dict(topk=topk, ranked=ranked)


# --------------------------------------------------------------------------
# landmark summary (upstream of the routed attention)
# --------------------------------------------------------------------------
def landmark_summary(qL, k, S: int, scale: Optional[float] = None):
    """Landmark key and entropy bias of every complete chunk (paperglide, "The
    HiLS-Attention Mechanism": the landmark query of a chunk scores the
    chunk's tokens, their softmax weights the keys into the summary key and
    the entropy of those weights is the bias; the overview calls this the
    first-order Taylor expansion of the chunk's attention mass).

    qL [B, Hkv, C, d] (one landmark query per chunk and KV head), k
    [B, Hkv, N, d]; C <= N // S. For chunk c with tokens t = cS .. cS+S-1:
      s_t = scale * qL_c . k_t,  p = softmax(s),
      kL_c = sum_t p_t k_t,      e_c = -sum_t p_t log p_t.
    Returns kL [B, Hkv, C, d] and e [B, Hkv, C] in float64."""
    qL = f64(qL)
    k = f64(k)
    B, Hkv, C, d = qL.shape
    sc = _scale(d, scale)
    kL = np.zeros((B, Hkv, C, d))
    e = np.zeros((B, Hkv, C))
    for b in range(B):
        for g in range(Hkv):
            for c in range(C):
                Kc = k[b, g, c * S:(c + 1) * S]
                s = sc * (Kc @ qL[b, g, c])
                logp = s - logsumexp(s)
                p = np.exp(logp)
                kL[b, g, c] = p @ Kc
                e[b, g, c] = -(p * logp).sum()
    return kL, e


def landmark_backward(qL, k, dkL, de, S: int, scale: Optional[float] = None):
    """Chain rule through landmark_summary (the pages print no backward; the
    gradient reaches the landmark query and the chunk's keys through both
    the summary key and the entropy). Per chunk, with s, p as above:
      dE/dp_t = dkL_c . k_t - de_c (log p_t + 1)
      dE/ds_t = p_t (dE/dp_t - sum_u p_u dE/dp_u)      (softmax backward)
      dqL_c   = scale sum_t dE/ds_t k_t
      dk_t    = scale dE/ds_t qL_c + p_t dkL_c          (through s and kL)
    Returns dqL [B, Hkv, C, d] and dk [B, Hkv, N, d] (zero past C S)."""
    qL = f64(qL)
    k = f64(k)
    dkL = f64(dkL)
    de = f64(de)
    B, Hkv, C, d = qL.shape
    sc = _scale(d, scale)
    dqL = np.zeros_like(qL)
    dk = np.zeros_like(k)
    for b in range(B):
        for g in range(Hkv):
            for c in range(C):
                Kc = k[b, g, c * S:(c + 1) * S]
                s = sc * (Kc @ qL[b, g, c])
                logp = s - logsumexp(s)
                p = np.exp(logp)
                dp = Kc @ dkL[b, g, c] - de[b, g, c] * (logp + 1.0)
                ds = p * (dp - p @ dp)
                dqL[b, g, c] = sc * (ds @ Kc)
                dk[b, g, c * S:(c + 1) * S] = sc * np.outer(ds, qL[b, g, c]) + np.outer(p, dkL[b, g, c])
    return dqL, dk


# --------------------------------------------------------------------------
# HoPE: partial rotary position encoding of queries and keys
# --------------------------------------------------------------------------
def hope_theta(d: int, base: float) -> np.ndarray:
    """Rotary frequencies theta_j = base^(-2j/d), j = 0 .. d/2 - 1 (the
    standard rotary schedule that HoPE starts from)."""
    return base ** (-2.0 * np.arange(d // 2) / d)


def hope_rotating(d: int, base: float, train_len: int) -> np.ndarray:
    """Which pairs keep their rotation (paperglide, "Implementation and
    Training Recipes", HoPE; dev.to, "Engineering Details", Hierarchical
    Positional Encoding): pair j rotates only if its period 2 pi / theta_j
    fits the training length; the others carry no position (NoPE)."""
    return 2.0 * math.pi / hope_theta(d, base) <= train_len


def hope_pairs(d: int, interleaved: bool):
    """Index arrays (a, b) of the rotation pairs: (j, j + d/2) by default,
    (2j, 2j + 1) when interleaved."""
    j = np.arange(d // 2)
    return (2 * j, 2 * j + 1) if interleaved else (j, j + d // 2)


def hope_rotate(x, pos=None, base: float = 10000.0, train_len: int = 8192,
                interleaved: bool = False, inverse: bool = False) -> np.ndarray:
    """Apply HoPE to x [B, H, N, d] at positions pos [B, N] (default: n).

    Every rotating pair (a, b) of row (b, h, n) is turned by the angle
    phi = pos * theta_j (by -phi when inverse, the transpose, which carries
    gradients back):
      y_a = x_a cos phi - x_b sin phi,  y_b = x_a sin phi + x_b cos phi;
    NoPE pairs are copied. Returns float64."""
    x = f64(x)
    B, H, N, d = x.shape
    if pos is None:
        pos = np.broadcast_to(np.arange(N), (B, N))
    pos = np.asarray(pos, dtype=np.float64)
    theta = hope_theta(d, base)
    rot = hope_rotating(d, base, train_len)
    a, b = hope_pairs(d, interleaved)
    y = x.copy()
    sign = -1.0 if inverse else 1.0
    for bi in range(B):
        phi = sign * np.outer(pos[bi], theta)            # [N, d/2]
        c = np.where(rot, np.cos(phi), 1.0)
        s = np.where(rot, np.sin(phi), 0.0)
        xa = x[bi][..., a]
        xb = x[bi][..., b]
        y[bi][..., a] = xa * c - xb * s
        y[bi][..., b] = xa * s + xb * c
    return y
