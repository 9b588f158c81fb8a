"""Degenerate sizes through every entry point: sequences shorter than a chunk
or than the window (no complete chunk, or no distant chunk for any query),
a single token, and a single-chunk cache. The method then reduces to causal
window attention (no chunk term), which the oracle computes directly."""
import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from workloads import Workload, make_inputs, make_landmark_inputs
from tests.hils_testutil import compare, fwd_parity, grad_tol, say, to_dev
from tests.test_gpu_decode import decode_parity, run_decode

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


@pytest.mark.parametrize("N", [1, 50, 64, 100, 191])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_short_sequences_forward_backward(N, dt):
    """N < W + S: no query has a distant chunk (and for N < 64 there is no
    complete chunk at all): forward = causal window attention, and the
    landmark gradients are zero."""
    lib = L()
    wl = Workload(f"short{N}", seed=41, dtype=dt, B=2, Hq=4, Hkv=2, d=64, N=N, S=64, K=4, W=128,
                  D=64 if dt == "bf16" else 0, r=32 if dt == "bf16" else 0, e_range=2.0,
                  mode="train")
    say(f"case short sequence N={N} {dt}")
    t = make_inputs(wl)
    td = to_dev(t)
    out = lib.hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                            h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"))
    torch.cuda.synchronize()
    assert bool((out[2] == -1).all())
    fwd_parity(t, out, wl.S, wl.K, wl.W, dt, label=f"short{N}")
    g = lib.hils_attn_bwd(td["q"], td["k"], td["v"], td["kL"], td["e"], out[0], out[1], out[2],
                          td["dO"], wl.S, wl.K, wl.W, h=td.get("h"), W_down=td.get("W_down"),
                          W_up=td.get("W_up"))
    torch.cuda.synchronize()
    ref = H.hils_backward(t, t["dO"], wl.S, wl.K, wl.W, forced_topk=out[2].cpu().numpy())
    for n in ("dq", "dk", "dv", "dkL", "de"):
        compare(f"short{N} {n}", g[n].cpu().double().numpy(), ref[n], dt, grad_tol(dt, ref[n]))
    if wl.r:
        for n in ("dW_down", "dW_up"):
            compare(f"short{N} {n}", g[n].cpu().double().numpy(), ref[n], dt, grad_tol(dt, ref[n]))
    assert float(g["dkL"].abs().max() if g["dkL"].numel() else 0.0) == 0.0


@pytest.mark.parametrize("lens", [[1, 1], [1, 64], [63, 64, 65]])
def test_decode_first_tokens(lens):
    """Decode at the very start of a sequence (one token, one chunk)."""
    wl = Workload("dec_first", seed=43, dtype="bf16", B=len(lens), Hq=8, Hkv=2, d=128, N=128, S=64,
                  K=4, W=64, e_range=2.0, mode="decode", seq_len=lens)
    say(f"case decode first tokens {lens}")
    t = make_inputs(wl)
    out = run_decode(wl, to_dev(t))
    torch.cuda.synchronize()
    decode_parity(wl, t, out, [(b, g) for b in range(wl.B) for g in range(wl.Hkv)], f"first{lens}")


@pytest.mark.parametrize("N", [10, 64, 130])
def test_landmark_few_or_no_chunks(N):
    """Keys shorter than a chunk: no landmark to build and nothing added to
    dk; one or two chunks: the oracle's values."""
    lib = L()
    wl = Workload("lm_short", seed=45, dtype="bf16", B=1, Hq=2, Hkv=2, d=64, N=N, S=64, K=1, W=1,
                  e_range=1.0, mode="train")
    t = make_landmark_inputs(wl)
    td = {k: v.cuda() for k, v in t.items()}
    kL, e, kL32, e32 = lib.hils_landmark_fwd(td["qL"], td["k"], 64, want_f32=True)
    dk0 = torch.ones(td["k"].shape, dtype=torch.float32, device="cuda")
    dqL, dk = lib.hils_landmark_bwd(td["qL"], td["k"], td["dkL"], td["de"], 64, dk=dk0.clone())
    torch.cuda.synchronize()
    C = N // 64
    assert kL.shape == (1, 2, C, 64) and e.shape == (1, 2, C)
    assert torch.equal(dk[:, :, C * 64:], dk0[:, :, C * 64:])
    if C:
        rkL, re = H.landmark_summary(t["qL"], t["k"], 64)
        rdq, rdk = H.landmark_backward(t["qL"], t["k"], t["dkL"], t["de"], 64)
        tol = dict(max_abs=2e-5, mean_abs=2e-6)
        compare("lm kL", kL32.cpu().double().numpy(), rkL, "bf16", tol)
        compare("lm e", e32.cpu().double().numpy(), re, "bf16", tol)
        compare("lm dqL", dqL.cpu().double().numpy(), rdq, "bf16", tol)
        compare("lm dk", (dk - dk0)[:, :, :C * 64].cpu().double().numpy(), rdk[:, :, :C * 64], "bf16", tol)


def _misaligned_like(t):
    """A contiguous int32 tensor of t's shape whose data starts 4 bytes past a
    16-byte boundary (a caller's buffer the kernels may not load or store as
    16-byte vectors)."""
    buf = torch.empty(t.numel() + 4, dtype=t.dtype, device=t.device)
    off = next(j for j in range(1, 4) if (buf.data_ptr() + 4 * j) % 16 != 0)
    m = buf[off:off + t.numel()].view(t.shape)
    assert m.data_ptr() % 16 != 0 and m.is_contiguous()
    return m


@pytest.mark.parametrize("strategy", ["union", "compact", "chunk_major"])
def test_misaligned_topk_idx_buffers(strategy):
    """K a multiple of 4 with a topk_idx buffer that is 4-byte but not 16-byte
    aligned: routing stores and the attention kernels read the ids one at a
    time instead of as 16-byte vectors. The selections equal those written to
    an aligned buffer; o and lse equal them bit for bit where the strategy
    sums in a fixed order (union, chunk-major) and match the oracle for the
    compacted strategy (its rows reach their buckets through atomic counters,
    so its sums are ordered by arrival); the backward with the misaligned ids
    (its query pass then takes the per-tile kernel) matches the oracle."""
    lib = L()
    sid = {"union": lib.FWD_UNION, "compact": lib.FWD_COMPACT, "chunk_major": lib.FWD_CHUNK_MAJOR}
    wl = Workload(f"mis_{strategy}", seed=47, dtype="bf16", B=1, Hq=4, Hkv=4, d=64, N=2048, S=64,
                  K=8, W=128, D=64, r=32, e_range=2.0, mode="train")
    say(f"case misaligned topk_idx, strategy {strategy}")
    t = make_inputs(wl)
    td = to_dev(t)
    args = (td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W)
    kw = dict(h=td["h"], W_down=td["W_down"], W_up=td["W_up"], strategy=sid[strategy])
    o0, lse0, idx0 = lib.hils_attn_fwd(*args, **kw)
    o1, lse1, idx1, ws = lib.fwd_buffers(td["q"], td["k"], wl.S, wl.K, wl.W, h=td["h"],
                                         W_down=td["W_down"], strategy=sid[strategy])
    idx_m = _misaligned_like(idx1)
    lib.hils_attn_fwd(*args, out=(o1, lse1, idx_m, ws), **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx_m, idx0)
    if strategy == "compact":
        fwd_parity(t, (o1, lse1, idx_m), wl.S, wl.K, wl.W, "bf16", label=f"misaligned {strategy}")
    else:
        assert torch.equal(o1, o0)
        assert torch.equal(lse1, lse0)
    g = lib.hils_attn_bwd(td["q"], td["k"], td["v"], td["kL"], td["e"], o0, lse0, idx_m, td["dO"],
                          wl.S, wl.K, wl.W, h=td["h"], W_down=td["W_down"], W_up=td["W_up"])
    torch.cuda.synchronize()
    ref = H.hils_backward(t, t["dO"], wl.S, wl.K, wl.W, forced_topk=idx0.cpu().numpy())
    for n in ("dq", "dk", "dv", "dkL", "de", "dW_down", "dW_up"):
        compare(f"misaligned {strategy} {n}", g[n].cpu().double().numpy(), ref[n], "bf16",
                grad_tol("bf16", ref[n]))
