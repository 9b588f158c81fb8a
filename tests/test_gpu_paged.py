"""Decode over a paged KV cache (page = chunk = 64 tokens) and decode steps
replayed from captured HIP graphs.

The paged cache is the contiguous one scattered into pages in a random order
(unused pages hold NaN, so a read of a wrong page shows). The paged step must
give the contiguous step's outputs bit for bit (same arithmetic, other
addresses) and the oracle's within the stated tolerance. A captured step is
replayed several times, with eager work and new query contents in between,
and every replay must equal an eager step on the same contents bit for bit."""
import pytest
import torch

from workloads import Workload, make_inputs
from tests.hils_testutil import say, to_dev
from tests.test_gpu_decode import decode_parity, run_decode

pytestmark = pytest.mark.gpu
S = 64


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def to_pages(td, seed=5, extra=7):
    """Pages [P, Hkv, S, d] of the contiguous caches in a random order, with
    the landmark rows and biases of each page, and the page table."""
    k, v, kL, e = td["k"], td["v"], td["kL"], td["e"]
    B, Hkv, N, d = k.shape
    maxp = N // S
    C = kL.shape[2]
    P = B * maxp + extra
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(P, generator=g)[:B * maxp].reshape(B, maxp).to(k.device)
    nan = float("nan")
    kp = torch.full((P, Hkv, S, d), nan, dtype=k.dtype, device=k.device)
    vp = torch.full_like(kp, nan)
    kp[perm] = k.reshape(B, Hkv, maxp, S, d).permute(0, 2, 1, 3, 4)
    vp[perm] = v.reshape(B, Hkv, maxp, S, d).permute(0, 2, 1, 3, 4)
    kLp = torch.full((P, Hkv, d), nan, dtype=kL.dtype, device=k.device)
    ep = torch.full((P, Hkv), nan, dtype=e.dtype, device=k.device)
    kLp[perm[:, :C]] = kL.permute(0, 2, 1, 3)
    ep[perm[:, :C]] = e.permute(0, 2, 1)
    return dict(k_pages=kp.contiguous(), v_pages=vp.contiguous(), kL_pages=kLp, e_pages=ep,
                page_table=perm.to(torch.int32).contiguous())


def run_paged(wl, td, pg, out=None):
    return L().hils_decode_paged(td["q"], pg["k_pages"], pg["v_pages"], pg["page_table"],
                                 td["seq_len"], pg["kL_pages"], pg["e_pages"], wl.S, wl.K, wl.W,
                                 h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"),
                                 out=out)


CASES = [
    # name, dtype, B, Hq, Hkv, d, Nk (a multiple of 64), K, W, D, r, seq_lens
    ("gqa4_d128", "bf16", 3, 16, 4, 128, 8192, 8, 512, 0, 0, [8192, 5000, 700]),
    ("mha_d64_qcal", "bf16", 2, 4, 4, 64, 20032, 16, 512, 128, 32, [20032, 13001]),
    ("gqa8_d128_k32", "bf16", 2, 16, 2, 128, 40000, 32, 1024, 0, 0, [40000, 39999]),
    ("gqa2_d64_short", "bf16", 4, 4, 2, 64, 3008, 4, 128, 0, 0, [3008, 64, 1, 200]),
    ("fp32_d64_qcal", "fp32", 2, 2, 1, 64, 6016, 5, 256, 64, 32, [6016, 4321]),
]


def wl_of(case, seed=23):
    name, dt, B, Hq, Hkv, d, Nk, K, W, D, r, lens = case
    return Workload(name, seed=seed, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=Nk, S=S, K=K, W=W, D=D,
                    r=r, e_range=2.0, e_shift=1.0, mode="decode", seq_len=lens)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_decode_equals_contiguous_and_oracle(case):
    wl = wl_of(case)
    say(f"case paged decode {wl.name}")
    t = make_inputs(wl)
    td = to_dev(t)
    pg = to_pages(td)
    ref = run_decode(wl, td)
    got = run_paged(wl, td, pg)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "topk_idx"), got, ref):
        assert torch.equal(a, b), f"{wl.name}: paged {name} differs from contiguous"
    pairs = [(b, g) for b in range(wl.B) for g in range(wl.Hkv)]
    decode_parity(wl, t, got, pairs, f"{wl.name} paged")


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_graph_replays_equal_eager(paged):
    lib = L()
    wl = wl_of(("graph_gqa4_qcal", "bf16", 2, 8, 2, 128, 12800, 8, 512, 128, 32, [12800, 7000]))
    say(f"case decode graph replay paged={paged}")
    td = to_dev(make_inputs(wl))
    pg = to_pages(td) if paged else None
    bufs = lib.decode_buffers(td["q"], td["k"], wl.S, wl.K, wl.W, td.get("h"), td.get("W_down"))

    def step(out):
        if paged:
            return run_paged(wl, td, pg, out=out)
        return L().hils_decode(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                               seq_len=td["seq_len"], h=td["h"], W_down=td["W_down"],
                               W_up=td["W_up"], out=out)

    step(bufs)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(bufs)
    gen = torch.Generator(device="cuda").manual_seed(9)
    for rep in range(4):
        if rep >= 2:  # new query contents in the captured input buffer
            td["q"].copy_(torch.randn(td["q"].shape, generator=gen, device="cuda").to(td["q"].dtype))
        graph.replay()
        torch.cuda.synchronize()
        got = tuple(x.clone() for x in bufs[:3])
        # eager work between replays: an eager step into fresh outputs
        want = step(None)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "topk_idx"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
    say("  4 replays equal the eager step")
