"""HoPE rotation (hils_hope) against the oracle: both pair layouts, both
directions, bf16 and fp32, d = 64 and 128, ragged sizes, positions from a
table up to 2^31 - 1, in place, the decode form (one position per sequence),
sampled rows of the 345M prefill query tensor, and the rotation in its place
on the path (landmark summary, routing, attention, backward) in fp32."""
import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from tests.hils_testutil import TOL, compare, say
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def check(name, got, ref, dt):
    """The method's tolerance, and for bf16 at most one rounding of the exact
    value (half an ulp, 2^-9 relative, plus the fp32 arithmetic)."""
    got = got.cpu().double().numpy()
    compare(name, got, ref, dt)
    if dt == "bf16":
        err = np.abs(got - ref)
        bound = np.abs(ref) * 2.0 ** -8 + 1e-6
        assert (err <= bound).all(), f"{name}: {int((err > bound).sum())} values beyond one bf16 rounding"


def rand(shape, dt, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    return x.to(torch.bfloat16) if dt == "bf16" else x


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("il", [False, True])
@pytest.mark.parametrize("inv", [False, True])
def test_hope_matches_oracle(dt, d, il, inv):
    lib = L()
    B, Hh, N = 2, 3, 37
    say(f"case hope {dt} d={d} interleaved={il} inverse={inv}")
    x = rand((B, Hh, N, d), dt, 11 + d)
    g = torch.Generator().manual_seed(5)
    pos = torch.randint(0, 1 << 24, (B, N), generator=g, dtype=torch.int32)
    pos[0, :4] = torch.tensor([0, 1, 2 ** 31 - 1, 2 ** 30 + 12345], dtype=torch.int32)
    for L_train in (8192, 100, 10 ** 7):
        y = lib.hils_hope(x.cuda(), pos.cuda(), base=10000.0, train_len=L_train, interleaved=il, inverse=inv)
        y0 = lib.hils_hope(x.cuda(), None, base=500000.0, train_len=L_train, interleaved=il, inverse=inv)
        torch.cuda.synchronize()
        ref = H.hope_rotate(x, pos.numpy(), 10000.0, L_train, interleaved=il, inverse=inv)
        ref0 = H.hope_rotate(x, None, 500000.0, L_train, interleaved=il, inverse=inv)
        check(f"hope L={L_train}", y, ref, dt)
        check(f"hope L={L_train} pos=n", y0, ref0, dt)
        # NoPE pairs are copied bit for bit
        rot = H.hope_rotating(d, 10000.0, L_train)
        a, b = H.hope_pairs(d, il)
        keep = np.concatenate([a[~rot], b[~rot]])
        assert torch.equal(y.cpu()[..., keep], x[..., keep])


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_hope_in_place_and_round_trip(dt):
    lib = L()
    say(f"case hope in place {dt}")
    x = rand((3, 5, 130, 64), dt, 21).cuda()
    pos = torch.randint(0, 1 << 20, (3, 130), dtype=torch.int32, generator=torch.Generator().manual_seed(2)).cuda()
    y = lib.hils_hope(x, pos, train_len=4096)
    z = x.clone()
    lib.hils_hope(z, pos, train_len=4096, out=z)
    torch.cuda.synchronize()
    assert torch.equal(y, z)
    back = lib.hils_hope(y, pos, train_len=4096, inverse=True)
    torch.cuda.synchronize()
    ref = H.hope_rotate(H.hope_rotate(x.cpu(), pos.cpu().numpy(), 1e4, 4096), pos.cpu().numpy(), 1e4, 4096,
                        inverse=True)
    np.testing.assert_allclose(ref, x.cpu().double().numpy(), atol=1e-12)
    # fp32: back = x to rounding; bf16: two roundings
    compare("round trip", back.cpu().double().numpy(), x.cpu().double().numpy(), dt,
            dict(max_abs=1e-5, mean_abs=1e-6) if dt == "fp32" else None)


def test_hope_decode_form_and_empty():
    """Decode rotates one new query per sequence at position seq_len - 1;
    an empty batch is a no-op."""
    lib = L()
    say("case hope decode form")
    q = rand((4, 8, 1, 128), "bf16", 31)
    seq = torch.tensor([[1], [64], [70000], [524288]], dtype=torch.int32)
    y = lib.hils_hope(q.cuda(), (seq - 1).cuda(), train_len=32768)
    torch.cuda.synchronize()
    check("decode", y, H.hope_rotate(q, (seq - 1).numpy(), 1e4, 32768), "bf16")
    e = torch.empty((0, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    assert lib.hils_hope(e).shape == e.shape


def test_hope_prefill_345m_sampled_rows():
    """The 345M prefill query tensor [4, 16, 8192, 64] (bf16) at positions n,
    training length 8192: sampled positions of every (batch, head) against
    the oracle."""
    lib = L()
    wl = WORKLOADS["prefill_345m"]
    say("case hope prefill_345m sampled rows")
    x = rand((wl.B, wl.Hq, wl.N, wl.d), "bf16", 41).cuda()
    y = lib.hils_hope(x, None, train_len=wl.N)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(0).choice(wl.N, 48, replace=False))
    idx[:2] = [0, wl.N - 1]
    idx = np.sort(idx)
    xs = x[:, :, idx].cpu()
    pos = np.broadcast_to(idx, (wl.B, len(idx)))
    ref = H.hope_rotate(xs, pos, 1e4, wl.N)
    check("prefill_345m rows", y[:, :, idx], ref, "bf16")


def test_hope_landmark_attention_chain_forward_and_backward():
    """The rotation in its place on the path (fp32): q and k rotated, the
    landmark summary built from the rotated keys, routing and attention on
    the rotated inputs; backward through attention, the landmark summary
    (added into dk) and the transposed rotation. Every stage's output against
    the same chain of oracle functions run on the original inputs."""
    from tests.hils_testutil import fwd_parity, grad_tol
    from workloads import Workload, make_inputs, make_landmark_inputs
    lib = L()
    Ltr = 512  # pairs 0 .. 15 rotate, 16 .. 31 carry no position
    wl = Workload("hope_chain", seed=51, dtype="fp32", B=1, Hq=4, Hkv=2, d=64, N=700, S=64, K=4, W=128,
                  D=64, r=16, e_range=2.0, mode="train")
    say("case hope + landmark + attention chain (fp32)")
    t = make_inputs(wl)
    qL = make_landmark_inputs(wl, keys=False)["qL"]
    # GPU chain
    dev = {n: x.cuda() for n, x in t.items() if isinstance(x, torch.Tensor)}
    q_r = lib.hils_hope(dev["q"], None, train_len=Ltr)
    k_r = lib.hils_hope(dev["k"], None, train_len=Ltr)
    kL, e = lib.hils_landmark_fwd(qL.cuda(), k_r, wl.S)
    out = lib.hils_attn_fwd(q_r, k_r, dev["v"], kL, e, wl.S, wl.K, wl.W, h=dev["h"],
                            W_down=dev["W_down"], W_up=dev["W_up"])
    g = lib.hils_attn_bwd(q_r, k_r, dev["v"], kL, e, out[0], out[1], out[2], dev["dO"], wl.S, wl.K,
                          wl.W, h=dev["h"], W_down=dev["W_down"], W_up=dev["W_up"])
    dqL, dk_r = lib.hils_landmark_bwd(qL.cuda(), k_r, g["dkL"], g["de"], wl.S, dk=g["dk"])
    dq = lib.hils_hope(g["dq"], None, train_len=Ltr, inverse=True)
    dk = lib.hils_hope(dk_r, None, train_len=Ltr, inverse=True)
    torch.cuda.synchronize()
    # oracle chain
    rq = H.hope_rotate(t["q"], None, 1e4, Ltr)
    rk = H.hope_rotate(t["k"], None, 1e4, Ltr)
    rkL, re = H.landmark_summary(qL, rk, wl.S)
    compare("chain q_r", q_r.cpu().double().numpy(), rq, "fp32")
    compare("chain kL", kL.cpu().double().numpy(), rkL, "fp32")
    compare("chain e", e.cpu().double().numpy(), re, "fp32")
    t2 = dict(t)
    t2.update(q=rq, k=rk, kL=rkL, e=re)
    fwd_parity(t2, out, wl.S, wl.K, wl.W, "fp32", label="chain fwd")
    ref = H.hils_backward(t2, t["dO"], wl.S, wl.K, wl.W, forced_topk=out[2].cpu().numpy())
    rdqL, rdk_lm = H.landmark_backward(qL, rk, ref["dkL"], ref["de"], wl.S)
    want = {"dq": H.hope_rotate(ref["dq"], None, 1e4, Ltr, inverse=True),
            "dk": H.hope_rotate(ref["dk"] + rdk_lm, None, 1e4, Ltr, inverse=True),
            "dv": ref["dv"], "dqL": rdqL, "dW_down": ref["dW_down"], "dW_up": ref["dW_up"]}
    got = {"dq": dq, "dk": dk, "dv": g["dv"], "dqL": dqL, "dW_down": g["dW_down"], "dW_up": g["dW_up"]}
    for n in want:
        compare(f"chain {n}", got[n].cpu().double().numpy(), want[n], "fp32", grad_tol("fp32", want[n]))
