"""One Q-Cal pair shared by all heads (W_down [r, D], W_up [d, r]): prefill
forward (both routing paths), backward with the tied-weight gradients, and
decode, against the oracle."""
import pytest
import torch

from oracle import hils_oracle as H
from workloads import Workload, make_inputs
from tests.hils_testutil import compare, fwd_parity, grad_tol, say, to_dev
from tests.test_gpu_decode import decode_parity, run_decode

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def shared(t):
    """The workload's inputs with the pair of head 0 shared by every head."""
    t = dict(t)
    t["W_down"] = t["W_down"][0].contiguous()
    t["W_up"] = t["W_up"][0].contiguous()
    return t


CASES = [
    # name, dtype, B, Hq, Hkv, d, N, K, W, D, r
    ("bf16_mha_r32_upath", "bf16", 2, 4, 4, 64, 800, 4, 128, 128, 32),
    ("bf16_gqa2_r16", "bf16", 1, 4, 2, 64, 700, 4, 128, 64, 16),
    ("fp32_gqa2_d128_r16", "fp32", 1, 4, 2, 128, 500, 4, 128, 64, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shared_qcal_forward_backward(case):
    name, dt, B, Hq, Hkv, d, N, K, W, D, r = case
    lib = L()
    wl = Workload(name, seed=61, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0, e_shift=1.0, mode="train")
    say(f"case shared Q-Cal {name}")
    t = shared(make_inputs(wl))
    td = to_dev(t)
    out = lib.hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                            h=td["h"], W_down=td["W_down"], W_up=td["W_up"])
    g = lib.hils_attn_bwd(td["q"], td["k"], td["v"], td["kL"], td["e"], out[0], out[1], out[2],
                          td["dO"], wl.S, wl.K, wl.W, h=td["h"], W_down=td["W_down"], W_up=td["W_up"],
                          want_dh=True)
    torch.cuda.synchronize()
    fwd_parity(t, out, wl.S, wl.K, wl.W, dt, label=name)
    ref = H.hils_backward(t, t["dO"], wl.S, wl.K, wl.W, forced_topk=out[2].cpu().numpy())
    assert g["dW_down"].shape == (r, D) and g["dW_up"].shape == (d, r)
    for n in ("dq", "dk", "dv", "dkL", "de", "dW_down", "dW_up", "dh"):
        compare(f"{name} {n}", g[n].cpu().double().numpy(), ref[n], dt, grad_tol(dt, ref[n]))


def test_shared_qcal_decode():
    wl = Workload("dec_shared", seed=63, dtype="bf16", B=3, Hq=8, Hkv=2, d=128, N=1024, S=64, K=4,
                  W=128, D=128, r=32, e_range=2.0, mode="decode", seq_len=[1024, 700, 333])
    say("case shared Q-Cal decode")
    t = shared(make_inputs(wl))
    out = run_decode(wl, to_dev(t))
    torch.cuda.synchronize()
    decode_parity(wl, t, out, [(b, g) for b in range(wl.B) for g in range(wl.Hkv)], "dec_shared")


def test_shared_qcal_paged_decode_equals_contiguous():
    """The paged entry point with a shared pair: bit for bit the contiguous
    decode, and the oracle."""
    from tests.test_gpu_paged import run_paged, to_pages
    wl = Workload("paged_shared", seed=65, dtype="bf16", B=2, Hq=4, Hkv=4, d=64, N=4096, S=64, K=8,
                  W=256, D=128, r=32, e_range=2.0, e_shift=1.0, mode="decode", seq_len=[4096, 2500])
    say("case shared Q-Cal paged decode")
    t = shared(make_inputs(wl))
    td = to_dev(t)
    pg = to_pages(td)
    ref = run_decode(wl, td)
    got = run_paged(wl, td, pg)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "topk_idx"), got, ref):
        assert torch.equal(a, b), f"paged {name} differs from contiguous"
    decode_parity(wl, t, got, [(b, g) for b in range(wl.B) for g in range(wl.Hkv)], "paged_shared")
