"""GPU parity of hils_decode against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from workloads import WORKLOADS, Workload, make_group_inputs, make_inputs
from tests.hils_testutil import check_topk_row, compare, say, to_dev

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def run_decode(wl, td):
    return L().hils_decode(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                           seq_len=td["seq_len"], h=td.get("h"), W_down=td.get("W_down"),
                           W_up=td.get("W_up"))


def oracle_ranked(t, b, g, S, K, W):
    """The oracle's ranking of the distant chunks of sequence b, group g
    (selection steps only: the caches are not read)."""
    r = H.hils_decode(t, S, K, W, batches=[b], groups=[g], rank_only=True)
    sel_sorted, order = r["ranked"][(b, g)]
    return sel_sorted, order, len(order)


def decode_parity(wl, t_cpu, out, pairs, label):
    o, lse, idx = (x.cpu() for x in out)
    idx = idx.numpy()
    G = wl.G
    nt = 0
    for (b, g) in pairs:
        sel_sorted, order, nd = oracle_ranked(t_cpu, b, g, wl.S, wl.K, wl.W)
        ok, tie = check_topk_row(idx[b, g], sel_sorted, order, wl.K, nd)
        nt += tie
        assert ok, f"{label}: topk mismatch b={b} g={g}: gpu={idx[b, g].tolist()} oracle={sorted(order[:wl.K].tolist())}"
    say(f"{label}: topk ok on {len(pairs)} (seq, kv-head) pairs ({nt} near-ties)")
    bs = sorted(set(b for b, _ in pairs))
    gs = sorted(set(g for _, g in pairs))
    ref = H.hils_decode(t_cpu, wl.S, wl.K, wl.W, batches=bs, groups=gs, forced_topk=idx)
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for (b, g) in pairs:
        hs = slice(g * G, (g + 1) * G)
        got_o.append(o[b, hs].double().numpy()); ref_o.append(ref["o"][b, hs])
        got_l.append(lse[b, hs].double().numpy()); ref_l.append(ref["lse"][b, hs])
    compare(f"{label} o", np.stack(got_o), np.stack(ref_o), wl.dtype)
    lt = 2e-3 if wl.dtype == "bf16" else 1e-5
    compare(f"{label} lse", np.stack(got_l), np.stack(ref_l), wl.dtype, dict(max_abs=lt, mean_abs=lt))


SMALL = [
    # name, dtype, B, Hq, Hkv, d, Nk, K, W, D, r, seq_lens, e_shift
    ("gqa4_d128", "bf16", 3, 16, 4, 128, 8192, 8, 512, 0, 0, [8192, 5000, 700], 0.0),
    ("mha_d64_qcal", "bf16", 2, 4, 4, 64, 20000, 16, 512, 128, 32, [20000, 13001], 3.0),
    ("gqa8_d128", "bf16", 2, 16, 2, 128, 40000, 32, 1024, 0, 0, [40000, 39999], 1.0),
    ("gqa2_d64_k4", "bf16", 4, 4, 2, 64, 3000, 4, 128, 0, 0, [3000, 64, 1, 200], 2.0),
    ("fp32_d64", "fp32", 2, 2, 1, 64, 6000, 5, 256, 64, 32, [6000, 4321], 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_decode_small(case):
    name, dt, B, Hq, Hkv, d, Nk, K, W, D, r, lens, sh = case
    wl = Workload(name, seed=21, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=Nk, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0, e_shift=sh, mode="decode", seq_len=lens)
    say(f"case decode {name}")
    t = make_inputs(wl)
    out = run_decode(wl, to_dev(t))
    torch.cuda.synchronize()
    pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    decode_parity(wl, t, out, pairs, name)


def test_decode_matches_prefill_last_row():
    """A decode at position n-1 equals row n-1 of the prefill on the same cache."""
    wlp = Workload("dp", seed=23, dtype="bf16", B=1, Hq=8, Hkv=2, d=128, N=3000, S=64, K=6, W=256,
                   D=64, r=32, e_range=2.0, e_shift=2.0)
    t = make_inputs(wlp)
    td = to_dev(t)
    o, lse, idx = L().hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], 64, 6, 256,
                                     h=td["h"], W_down=td["W_down"], W_up=td["W_up"])
    n = 3000
    od, ld, idd = L().hils_decode(td["q"][:, :, n - 1].contiguous(), td["k"], td["v"], td["kL"],
                                  td["e"], 64, 6, 256,
                                  seq_len=torch.tensor([n], dtype=torch.int32, device="cuda"),
                                  h=td["h"][:, n - 1].contiguous(), W_down=td["W_down"],
                                  W_up=td["W_up"])
    torch.cuda.synchronize()
    assert torch.equal(idd.cpu(), idx[:, :, n - 1].cpu())
    err = (od.float() - o[:, :, n - 1].float()).abs().max().item()
    say(f"decode vs prefill row: max |diff| {err:.3e}")
    assert err < 1e-2
    assert (ld - lse[:, :, n - 1]).abs().max().item() < 1e-4


def big_decode_case(name, pairs):
    wl = WORKLOADS[name]
    say(f"case decode {name} full size: generating inputs on the GPU")
    t = make_inputs(wl, device="cuda")
    out = run_decode(wl, t)
    torch.cuda.synchronize()
    o, lse, idx = (x.cpu() for x in out)
    say(f"{name}: ran; checking {pairs}")
    for (b, g) in pairs:
        n = int(t["seq_len"][b])
        # selection from landmarks only (no K/V needed)
        tg = make_group_inputs(wl, b, g, kv_rows=[])
        assert torch.equal(tg["kL"][0, 0], t["kL"][b, g].cpu())
        sel_sorted, order, nd = oracle_ranked(tg, 0, 0, wl.S, wl.K, wl.W)
        ok, tie = check_topk_row(idx[b, g], sel_sorted, order, wl.K, nd)
        assert ok, f"{name}: topk mismatch b={b} g={g}"
        # regenerate only the selected chunks and the window, then check o / lse
        rows = [j for c in idx[b, g].tolist() if c >= 0 for j in range(c * wl.S, (c + 1) * wl.S)]
        rows += list(range(nd * wl.S, n))
        tg = make_group_inputs(wl, b, g, kv_rows=rows)
        ref = H.hils_decode(tg, wl.S, wl.K, wl.W, forced_topk=idx[b:b + 1, g:g + 1].numpy())
        G = wl.G
        compare(f"{name} b={b} g={g} o", o[b, g * G:(g + 1) * G].double().numpy(), ref["o"][0], wl.dtype)
        compare(f"{name} b={b} g={g} lse", lse[b, g * G:(g + 1) * G].double().numpy(), ref["lse"][0],
                wl.dtype, dict(max_abs=2e-3, mean_abs=2e-3))
    return wl, idx


def test_decode_7b_512k_full_size_sampled():
    big_decode_case("decode_7b_512k", [(0, 0), (17, 5), (31, 7)])


def test_decode_4m_full_size_needle():
    wl, idx = big_decode_case("decode_4m", [(0, 0), (0, 9), (0, 15)])
    from workloads import needle_chunk_decode
    for g in range(wl.Hkv):
        assert needle_chunk_decode(wl, 0, g) in idx[0, g].tolist(), f"needle not selected for head {g}"
    say("decode_4m: every head selected its planted needle chunk")
