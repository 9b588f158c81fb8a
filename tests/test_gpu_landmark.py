"""GPU parity of the landmark summary (hils_landmark_fwd / hils_landmark_bwd)
against the fp64 oracle's landmark_summary / landmark_backward."""
import math

import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from workloads import WORKLOADS, Workload, make_landmark_inputs
from tests.hils_testutil import compare, say

pytestmark = pytest.mark.gpu

S = 64


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def wl_of(name, dt, B, Hkv, d, N, seed=51):
    return Workload(name, seed=seed, dtype=dt, B=B, Hq=Hkv, Hkv=Hkv, d=d, N=N, S=S, K=4, W=128,
                    D=0, r=0, e_range=1.0, mode="train")


CASES = [
    # name, dtype, B, Hkv, d, N (N not a multiple of S: a ragged tail of keys)
    ("bf16_d64", "bf16", 2, 3, 64, 1000),
    ("bf16_d128", "bf16", 1, 2, 128, 700),
    ("fp32_d64", "fp32", 1, 2, 64, 640),
    ("fp32_d128", "fp32", 2, 1, 128, 300),
]


def run_fwd_bwd(t, dk0=None):
    lib = L()
    kL, e, kL32, e32 = lib.hils_landmark_fwd(t["qL"], t["k"], S, want_f32=True)
    dk = None if dk0 is None else dk0.clone()
    dqL, dk = lib.hils_landmark_bwd(t["qL"], t["k"], t["dkL"], t["de"], S, dk=dk)
    torch.cuda.synchronize()
    return kL, e, kL32, e32, dqL, dk


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_landmark_parity(case):
    name, dt, B, Hkv, d, N = case
    wl = wl_of(name, dt, B, Hkv, d, N)
    say(f"case landmark {name}")
    t = make_landmark_inputs(wl)
    td = {k: v.cuda() for k, v in t.items()}
    # dk arrives holding other gradients: the keys' part is added to it
    dk0 = torch.randn(t["k"].shape, generator=torch.Generator().manual_seed(7)).cuda()
    kL, e, kL32, e32, dqL, dk = run_fwd_bwd(td, dk0)
    rkL, re = H.landmark_summary(t["qL"], t["k"], S)
    rdq, rdk = H.landmark_backward(t["qL"], t["k"], t["dkL"], t["de"], S)
    # the fp32 results carry only fp32 rounding (the inputs are the same values)
    tol = dict(max_abs=2e-5, mean_abs=2e-6)
    compare(f"{name} kL", kL32.cpu().double().numpy(), rkL, dt, tol)
    compare(f"{name} e", e32.cpu().double().numpy(), re, dt, tol)
    compare(f"{name} dqL", dqL.cpu().double().numpy(), rdq, dt, tol)
    C = N // S
    got_dk = (dk - dk0).cpu().double().numpy()
    compare(f"{name} dk", got_dk[:, :, :C * S], rdk[:, :, :C * S], dt, tol)
    # keys past the last complete chunk are not touched, bit for bit
    assert torch.equal(dk[:, :, C * S:].cpu(), dk0[:, :, C * S:].cpu())
    # the outputs in the problem dtype are the fp32 values rounded to nearest even
    assert torch.equal(kL, kL32.to(kL.dtype)) and torch.equal(e, e32.to(e.dtype))


def test_landmark_degenerate_chunks():
    """Uniform chunks (every key equal): kL is that key and e = ln S; a
    landmark query far along one key of an orthonormal chunk: one-hot
    weights, kL that key, e ~ 0 and gradients that vanish in the queries."""
    lib = L()
    d, N = 64, 4 * S
    g = torch.Generator().manual_seed(3)
    k = torch.randn(1, 1, N, d, generator=g)
    k[0, 0, :S] = k[0, 0, 5]                      # chunk 0: uniform
    k[0, 0, S:2 * S] = torch.eye(S, d)            # chunk 1: orthonormal keys
    qL = torch.randn(1, 1, N // S, d, generator=g)
    qL[0, 0, 1] = 300.0 * torch.eye(S, d)[9]      # chunk 1: aimed at key 9
    qL[0, 0, 2] = 0.0                             # chunk 2: zero query -> uniform weights
    dkL = torch.randn(1, 1, N // S, d, generator=g)
    de = torch.randn(1, 1, N // S, generator=g)
    t = dict(qL=qL.cuda(), k=k.cuda(), dkL=dkL.cuda(), de=de.cuda())
    kL, e, kL32, e32, dqL, dk = run_fwd_bwd(t)
    rkL, re = H.landmark_summary(qL, k, S)
    rdq, rdk = H.landmark_backward(qL, k, dkL, de, S)
    tol = dict(max_abs=2e-5, mean_abs=2e-6)
    compare("degenerate kL", kL32.cpu().double().numpy(), rkL, "fp32", tol)
    compare("degenerate e", e32.cpu().double().numpy(), re, "fp32", tol)
    compare("degenerate dqL", dqL.cpu().double().numpy(), rdq, "fp32", tol)
    compare("degenerate dk", dk.cpu().double().numpy(), rdk, "fp32", tol)
    assert abs(float(e32[0, 0, 0]) - math.log(S)) < 1e-5
    assert abs(float(e32[0, 0, 2]) - math.log(S)) < 1e-5
    assert float(e32[0, 0, 1]) < 1e-5
    torch.testing.assert_close(kL32[0, 0, 1].cpu(), torch.eye(S, d)[9], atol=1e-6, rtol=0)


def test_landmark_train_shape_sampled_and_taylor_point():
    """The 345M training shape (B 8, 16 KV heads, N 8192, d 64, bf16): sampled
    chunks against the oracle, and at every chunk the surrogate at its own
    landmark query equals the chunk's exact log-mass (computed here in fp64
    from the same keys)."""
    wl = WORKLOADS["train_345m"]
    say("case landmark train_345m sampled")
    t = make_landmark_inputs(wl, device="cuda")
    kL, e, kL32, e32, dqL, dk = run_fwd_bwd(t)
    sc = 1 / math.sqrt(wl.d)
    C = wl.N // S
    # Taylor point, all chunks: scale qL.kL + e == logsumexp(scale qL.k_t)
    kc = t["k"].double().reshape(wl.B, wl.Hkv, C, S, wl.d)
    q64 = t["qL"].double()
    exact = torch.logsumexp(sc * torch.einsum("bgcsd,bgcd->bgcs", kc, q64), -1)
    sur = sc * (q64 * kL32.double()).sum(-1) + e32.double()
    err = (sur - exact).abs()
    say(f"  taylor point: max {float(err.max()):.2e} mean {float(err.mean()):.2e}")
    assert float(err.max()) < 1e-4 and float(err.mean()) < 1e-5
    # sampled chunks against the oracle
    rng = np.random.default_rng(11)
    for _ in range(6):
        b, g, c = int(rng.integers(wl.B)), int(rng.integers(wl.Hkv)), int(rng.integers(C))
        sl = (slice(b, b + 1), slice(g, g + 1))
        qs = t["qL"][sl][:, :, c:c + 1].cpu()
        ks = t["k"][sl][:, :, c * S:(c + 1) * S].cpu()
        rkL, re = H.landmark_summary(qs, ks, S)
        rdq, rdk = H.landmark_backward(qs, ks, t["dkL"][sl][:, :, c:c + 1].cpu(),
                                       t["de"][sl][:, :, c:c + 1].cpu(), S)
        tol = dict(max_abs=2e-5, mean_abs=2e-6)
        compare(f"({b},{g},{c}) kL", kL32[sl][:, :, c:c + 1].cpu().double().numpy(), rkL, "bf16", tol)
        compare(f"({b},{g},{c}) e", e32[sl][:, :, c:c + 1].cpu().double().numpy(), re, "bf16", tol)
        compare(f"({b},{g},{c}) dqL", dqL[sl][:, :, c:c + 1].cpu().double().numpy(), rdq, "bf16", tol)
        compare(f"({b},{g},{c}) dk", dk[sl][:, :, c * S:(c + 1) * S].cpu().double().numpy(), rdk,
                "bf16", tol)
