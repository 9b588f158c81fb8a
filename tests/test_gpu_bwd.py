"""GPU parity of hils_attn_bwd against the fp64 oracle's chain-rule backward."""
import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from workloads import WORKLOADS, Workload, make_group_inputs, make_inputs
from tests.hils_testutil import compare, grad_tol, say, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dkL", "de")
WGRADS = ("dW_down", "dW_up", "dh")


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def gpu_fwd_bwd(wl, td, want_dh=True):
    lib = L()
    o, lse, idx = lib.hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                                    h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"))
    g = lib.hils_attn_bwd(td["q"], td["k"], td["v"], td["kL"], td["e"], o, lse, idx, td["dO"], wl.S,
                          wl.K, wl.W, h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"),
                          want_dh=want_dh and "h" in td)
    torch.cuda.synchronize()
    return o, lse, idx, g


def tol(dt):
    return None


SMALL = [
    # name, dtype, B, Hq, Hkv, d, N, K, W, D, r, e_shift
    ("mha_d64_qcal", "bf16", 2, 2, 2, 64, 1000, 4, 128, 64, 32, 2.0),
    ("gqa4_d128_qcal", "bf16", 1, 8, 2, 128, 1100, 6, 256, 128, 32, 3.0),
    ("gqa2_d64", "bf16", 1, 4, 2, 64, 900, 5, 192, 0, 0, 8.0),
    ("fp32_d64_qcal", "fp32", 1, 2, 1, 64, 600, 3, 64, 64, 32, 1.0),
    # bf16 d = 64 with K a multiple of 4: the shared-block dq pass (G = 2, 4)
    ("gqa2_d64_k8_qcal", "bf16", 1, 4, 2, 64, 1300, 8, 192, 64, 16, 2.0),
    ("gqa4_d64_k4", "bf16", 1, 8, 2, 64, 800, 4, 128, 0, 0, 3.0),
    ("fp32_d128_gqa2_r16", "fp32", 1, 4, 2, 128, 500, 4, 128, 64, 16, 1.0),
    # Hq r and D multiples of 128: dW_down on the token-major weight-gradient
    # GEMM (two K splits summed in bf16; one split written directly in fp32)
    ("mha4_d64_qcal_wgemm", "bf16", 2, 4, 4, 64, 1024, 8, 128, 256, 32, 2.0),
    ("fp32_gqa2_qcal_wgemm", "fp32", 1, 4, 2, 64, 1024, 4, 128, 128, 32, 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_small(case):
    name, dt, B, Hq, Hkv, d, N, K, W, D, r, sh = case
    wl = Workload(name, seed=31, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0, e_shift=sh, mode="train")
    say(f"case bwd {name}")
    t = make_inputs(wl)
    o, lse, idx, g = gpu_fwd_bwd(wl, to_dev(t))
    ref = H.hils_backward(t, t["dO"], wl.S, wl.K, wl.W, forced_topk=idx.cpu().numpy())
    names = GRADS + (WGRADS if r else ())
    for n in names:
        compare(f"{name} {n}", g[n].cpu().double().numpy(), ref[n], dt, grad_tol(dt, ref[n]))


def test_bwd_extreme_token_scores():
    """Keys of some distant chunks scaled up, so that their token scores sit
    far above the rows' L (exp against L overflows; the dq pass redoes those
    row blocks against the chunk maximum). Gradients then reach magnitudes
    of tens, so the bf16 tolerance is applied relative to each gradient's
    largest oracle value."""
    wl = Workload("bwd_extreme", seed=33, dtype="bf16", B=1, Hq=2, Hkv=2, d=64, N=1000, S=64, K=4,
                  W=128, D=0, r=0, e_range=2.0, e_shift=4.0, mode="train")
    say("case bwd extreme token scores")
    t = make_inputs(wl)
    kk = t["k"].float()
    kk[:, :, 128:384] *= 45.0
    t["k"] = kk.to(torch.bfloat16)
    o, lse, idx, g = gpu_fwd_bwd(wl, to_dev(t))
    ref = H.hils_backward(t, t["dO"], wl.S, wl.K, wl.W, forced_topk=idx.cpu().numpy())
    for n in GRADS:
        sc = max(1.0, float(np.abs(ref[n]).max()))
        compare(f"extreme {n}", g[n].cpu().double().numpy() / sc, ref[n] / sc, "bf16")


def test_bwd_train_345m_full_size_sampled_groups():
    wl = WORKLOADS["train_345m"]
    say("case bwd train_345m full size")
    t = make_inputs(wl, device="cuda")
    o, lse, idx, g = gpu_fwd_bwd(wl, t, want_dh=False)
    idx = idx.cpu().numpy()
    for (b, h) in [(0, 0), (5, 11)]:
        tg = make_group_inputs(wl, b, h)
        assert torch.equal(tg["dO"][0], t["dO"][b, h:h + 1].cpu())
        ref = H.hils_backward(tg, tg["dO"], wl.S, wl.K, wl.W, forced_topk=idx[b:b + 1, h:h + 1])
        for n, sl in (("dq", (b, slice(h, h + 1))), ("dk", (b, slice(h, h + 1))),
                      ("dv", (b, slice(h, h + 1))), ("dkL", (b, slice(h, h + 1))),
                      ("de", (b, slice(h, h + 1)))):
            compare(f"train_345m b={b} h={h} {n}", g[n][sl].cpu().double().numpy(), ref[n][0], "bf16")


def test_bwd_train_345m_qcal_weight_grads_batch_slice():
    """The Q-Cal weight gradients of head h sum over every batch element; on a
    one-sequence slice of the workload they equal the oracle on group (0, h)."""
    wl = WORKLOADS["train_345m"].with_(B=1)
    t = make_inputs(wl, device="cuda")
    o, lse, idx, g = gpu_fwd_bwd(wl, t, want_dh=True)
    idx = idx.cpu().numpy()
    for h in (0, 9):
        tg = make_group_inputs(wl, 0, h)
        ref = H.hils_backward(tg, tg["dO"], wl.S, wl.K, wl.W, forced_topk=idx[:, h:h + 1])
        compare(f"train_345m[B=1] h={h} dW_down", g["dW_down"][h].cpu().double().numpy(), ref["dW_down"][0], "bf16")
        compare(f"train_345m[B=1] h={h} dW_up", g["dW_up"][h].cpu().double().numpy(), ref["dW_up"][0], "bf16")


DET = [
    # bucketed dq pass (d = 128, grouped heads), shared-block dq pass (d = 64
    # bf16), fp32, Q-Cal weight gradients
    ("det_gqa4_d128_qcal", "bf16", 1, 8, 2, 128, 3000, 8, 256, 128, 32, 1.0),
    ("det_mha_d64_qcal", "bf16", 2, 2, 2, 64, 2000, 8, 128, 128, 32, 2.0),
    ("det_fp32_gqa2_d64", "fp32", 1, 4, 2, 64, 1500, 5, 128, 64, 16, 1.0),
]


@pytest.mark.parametrize("case", DET, ids=[c[0] for c in DET])
def test_bwd_reruns_are_bit_identical(case):
    """Two backward calls on the same inputs give the same bits: the inverse
    index is a stable sort, the dq pass assigns chunks to waves statically
    and adds each row's chunk terms in slot order."""
    name, dt, B, Hq, Hkv, d, N, K, W, D, r, sh = case
    wl = Workload(name, seed=37, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0, e_shift=sh, mode="train")
    say(f"case bwd determinism {name}")
    td = to_dev(make_inputs(wl))
    lib = L()
    o, lse, idx = lib.hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                                    h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"))
    runs = []
    for _ in range(2):
        g = lib.hils_attn_bwd(td["q"], td["k"], td["v"], td["kL"], td["e"], o, lse, idx, td["dO"],
                              wl.S, wl.K, wl.W, h=td.get("h"), W_down=td.get("W_down"),
                              W_up=td.get("W_up"), want_dh=True)
        torch.cuda.synchronize()
        runs.append({n: v.clone() for n, v in g.items()})
    for n in GRADS:
        assert torch.equal(runs[0][n], runs[1][n]), f"{name}: {n} differs between runs"
    same_w = {n: torch.equal(runs[0][n], runs[1][n]) for n in runs[0] if n not in GRADS}
    say(f"  {name}: dq dk dv dkL de bit-identical; weight gradients identical: {same_w}")
