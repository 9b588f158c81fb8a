"""GPU parity of hils_route / hils_attn_fwd against the fp64 oracle."""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, Workload, make_inputs
from tests.hils_testutil import fwd_parity, say, to_dev, check_topk_row
from oracle import hils_oracle as H

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def run_fwd(wl, t):
    lib = L()
    td = to_dev(t)
    return lib.hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                             h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"))


SMALL = [
    # name, dtype, B, Hq, Hkv, d, N, K, W, D, r, e_shift
    ("mha_d64_qcal", "bf16", 2, 2, 2, 64, 1000, 4, 128, 64, 32, 0.0),
    ("mha_d64_chunkdom", "bf16", 1, 2, 2, 64, 1100, 6, 128, 0, 0, 8.0),
    ("gqa2_d128", "bf16", 1, 4, 2, 128, 900, 5, 192, 96, 16, 3.0),
    ("gqa4_d128_qcal", "bf16", 1, 8, 2, 128, 1300, 8, 256, 128, 32, 0.0),
    ("gqa4_d64_r64", "bf16", 1, 4, 1, 64, 777, 3, 64, 64, 64, 2.0),
    ("fp32_d64", "fp32", 1, 2, 1, 64, 700, 4, 128, 0, 0, 4.0),
    ("fp32_d64_qcal_gqa2", "fp32", 1, 4, 2, 64, 520, 3, 64, 64, 32, 1.0),
    ("fp32_d128_gqa4", "fp32", 1, 8, 2, 128, 450, 3, 64, 0, 0, 2.0),
    # selections spread over many chunks relative to a tile's slots: these
    # take the chunk-major strategy by default ((128 / G) * K < 4 * N / 64)
    ("spread_gqa4_d128_qcal", "bf16", 1, 8, 2, 128, 2300, 4, 256, 64, 32, 2.0),
    ("spread_mha_d64_fp32", "fp32", 1, 2, 2, 64, 4500, 2, 128, 0, 0, 3.0),
    ("spread_gqa2_d64_qcal", "bf16", 1, 4, 2, 64, 3000, 2, 192, 64, 16, 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small_all_rows(case):
    name, dt, B, Hq, Hkv, d, N, K, W, D, r, sh = case
    wl = Workload(name, seed=11, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0, e_shift=sh)
    say(f"case {name}")
    t = make_inputs(wl)
    out = run_fwd(wl, t)
    torch.cuda.synchronize()
    fwd_parity(t, out, wl.S, wl.K, wl.W, dt, label=name)


def test_fwd_extreme_token_scores():
    """Keys of some distant chunks scaled up (token scores far above the
    window's: exp2 against the window maximum overflows) and keys of the
    last tokens scaled up (window maxima far above the distant chunks'
    scores: the chunk probabilities underflow); both take the exact
    per-chunk maximum instead."""
    wl = Workload("extreme", seed=12, dtype="bf16", B=1, Hq=2, Hkv=2, d=64, N=1100, S=64, K=6, W=128,
                  D=0, r=0, e_range=2.0, e_shift=6.0)
    say("case extreme token scores")
    t = make_inputs(wl)
    k = t["k"].float()
    k[:, :, 128:384] *= 45.0
    k[:, :, 1004:] *= 45.0
    t["k"] = k.to(torch.bfloat16)
    out = run_fwd(wl, t)
    torch.cuda.synchronize()
    fwd_parity(t, out, wl.S, wl.K, wl.W, "bf16", label="extreme")


def test_fwd_tiny_workload():
    wl = WORKLOADS["tiny"]
    say("case tiny (fp32, needle chunk 7)")
    t = make_inputs(wl)
    out = run_fwd(wl, t)
    torch.cuda.synchronize()
    idx = out[2].cpu().numpy()
    assert 7 in idx[0, 0, wl.N - 1]
    fwd_parity(t, out, wl.S, wl.K, wl.W, "fp32", label="tiny")


@pytest.mark.parametrize("G,d,r,K", [
    (4, 128, 32, 6),    # GQA: fp32 calibrated queries, per-head scores in routing's epilogue
    (2, 64, 64, 12),    # two heads per group, rank 64
    (4, 64, 64, 6),     # four heads per group, d = 64
    (2, 128, 32, 20),   # K > 16 with grouped heads
    (1, 64, 32, 6),     # one head per KV group, bf16, rank 32: folded
    (1, 128, 64, 12),   # the same with rank 64 and d = 128
    (1, 64, 32, 20),    # K > 16: fp32 calibrated queries with one head per group
    (2, 64, 0, 6),      # no Q-Cal
])
def test_route_scores_match_oracle(G, d, r, K):
    """The selected chunks' per-head scores that routing returns (the fusion
    reads them) against the oracle's surrogate scores, within 2e-5."""
    wl = Workload("route", seed=5, dtype="bf16", B=1, Hq=2 * G, Hkv=2, d=d, N=1200, S=64, K=K,
                  W=128, D=64 if r else 0, r=r, e_range=2.0)
    t = make_inputs(wl)
    td = to_dev(t)
    idx, sc = L().hils_route(td["q"], td["kL"], td["e"], wl.S, wl.K, wl.W, h=td.get("h"),
                             W_down=td.get("W_down"), W_up=td.get("W_up"), with_scores=True)
    idx = idx.cpu().numpy()
    sc = sc.cpu().numpy()
    P = H.Problem(t, wl.S, wl.K, wl.W)
    err = 0.0
    n = 0
    for g in range(wl.Hkv):
        hs = slice(g * G, (g + 1) * G)
        for i in range(0, wl.N, 7):
            qh, _ = P.qhat_row(0, g, i, P.q[0, hs, i])
            s_ref, _ = H.surrogate_scores(qh, P.kL[0, g], P.e[0, g], H.n_distant(i, wl.W, wl.S),
                                          P.scale)
            for kk in range(wl.K):
                c = idx[0, g, i, kk]
                if c < 0:
                    assert np.all(np.isnan(sc[0, hs, i, kk]))
                    continue
                err = max(err, float(np.abs(sc[0, hs, i, kk] - s_ref[:, c]).max()))
                n += 1
    say(f"route scores G{G} d{d} r{r} K{K}: {n} checked, max abs err {err:.3e}")
    assert n > 0 and err < 2e-5


# one head per KV group over 625-938 distant chunks: routing's long-scan
# selection (every position's candidates in its own lane, buffered against
# its running K-th score), on both scoring paths (fp32 calibrated queries;
# bf16 with Q-Cal folded into routing), d = 64 and 128, K up to 32
LONG_SCAN = [
    # name, dtype, d, N, K, W, D, r
    ("ls_bf16_d64_k32", "bf16", 64, 40000, 32, 512, 64, 32),
    ("ls_bf16_d64_k8_u", "bf16", 64, 41000, 8, 256, 64, 32),
    ("ls_bf16_d128_k16_u", "bf16", 128, 60000, 16, 1024, 64, 64),
    ("ls_fp32_d64_k16", "fp32", 64, 40000, 16, 512, 0, 0),
    ("ls_bf16_d128_k4", "bf16", 128, 44000, 4, 128, 0, 0),
]


@pytest.mark.parametrize("case", LONG_SCAN, ids=[c[0] for c in LONG_SCAN])
def test_fwd_long_scan_sampled_rows(case):
    name, dt, d, N, K, W, D, r = case
    wl = Workload(name, seed=21, dtype=dt, B=1, Hq=2, Hkv=2, d=d, N=N, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0)
    say(f"case {name}")
    t = make_inputs(wl)
    out = run_fwd(wl, t)
    torch.cuda.synchronize()
    fwd_parity(t, out, wl.S, wl.K, wl.W, dt, rows=sample_rows(wl, 150), label=name)


def group_parity(wl, t_gpu, out, groups, rows, label):
    """Full-size run checked group by group: the oracle regenerates the
    (b, g) slabs on the CPU (bit-identical to the GPU's inputs) and checks
    the sampled rows."""
    from workloads import make_group_inputs
    o, lse, idx = out
    G = wl.G
    for (b, g) in groups:
        tg = make_group_inputs(wl, b, g, h_rows=rows)
        # the generator is device independent: the GPU inputs of this group match
        assert torch.equal(t_gpu["q"][b, g * G:(g + 1) * G].cpu(), tg["q"][0])
        assert torch.equal(t_gpu["k"][b, g].cpu(), tg["k"][0, 0])
        assert torch.equal(t_gpu["kL"][b, g].cpu(), tg["kL"][0, 0])
        sub = (o[b:b + 1, g * G:(g + 1) * G], lse[b:b + 1, g * G:(g + 1) * G], idx[b:b + 1, g:g + 1])
        fwd_parity(tg, sub, wl.S, wl.K, wl.W, wl.dtype, rows=rows, label=f"{label} b={b} g={g}")


def sample_rows(wl, n):
    N, W, S = wl.N, wl.W, wl.S
    edge = [0, 1, W - 2, W - 1, W, W + S - 2, W + S - 1, W + S, W + 2 * S, N - 65, N - 64, N - 2, N - 1]
    step = max(1, N // n)
    return sorted(set([i for i in edge if 0 <= i < N] + list(range(7, N, step))))


def test_fwd_prefill_345m_full_size_sampled():
    wl = WORKLOADS["prefill_345m"]
    say("case prefill_345m full size")
    t = make_inputs(wl, device="cuda")
    out = L().hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W, h=t["h"],
                            W_down=t["W_down"], W_up=t["W_up"])
    torch.cuda.synchronize()
    out = tuple(x.cpu() for x in out)
    group_parity(wl, t, out, [(0, 0), (3, 15), (1, 6)], sample_rows(wl, 160), "prefill_345m")


def test_fwd_prefill_1p4b_full_size_sampled():
    wl = WORKLOADS["prefill_1p4b"]
    say("case prefill_1p4b full size")
    t = make_inputs(wl, device="cuda")
    out = L().hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W, h=t["h"],
                            W_down=t["W_down"], W_up=t["W_up"])
    torch.cuda.synchronize()
    out = tuple(x.cpu() for x in out)
    del t["h"]
    group_parity(wl, t, out, [(0, 0), (0, 7)], sample_rows(wl, 60), "prefill_1p4b")
