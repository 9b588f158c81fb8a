"""hils_decode_noalloc (the decode entry point that allocates nothing: its
scratch is a static per-GPU buffer) against hils_decode with a caller
workspace: two calls in a row on the same buffer, the second smaller, each
equal to the workspace path bit for bit (same kernels, same inputs), and
within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

from oracle import hils_oracle as H
from workloads import Workload, make_inputs
from tests.hils_testutil import compare, say, to_dev

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


CASES = [
    # the larger call first, then a smaller one on the same static buffer
    Workload("noalloc_gqa4_d128_qcal", seed=41, dtype="bf16", B=3, Hq=16, Hkv=4, d=128, N=20000,
             S=64, K=16, W=512, D=128, r=32, e_range=2.0, e_shift=1.0, mode="decode",
             seq_len=[20000, 13333, 4097]),
    Workload("noalloc_mha_d64", seed=43, dtype="bf16", B=1, Hq=4, Hkv=4, d=64, N=3000, S=64,
             K=8, W=256, e_range=2.0, e_shift=2.0, mode="decode", seq_len=[2999]),
]


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    lib = L()
    for wl in CASES:
        say(f"case noalloc {wl.name}")
        t = make_inputs(wl)
        td = to_dev(t)
        args = (td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W)
        kw = dict(seq_len=td["seq_len"], h=td.get("h"), W_down=td.get("W_down"),
                  W_up=td.get("W_up"))
        ref = lib.hils_decode(*args, **kw)
        # preallocated outputs: the call itself allocates nothing
        out = (torch.full_like(ref[0], float("nan")), torch.full_like(ref[1], float("nan")),
               torch.full_like(ref[2], -7))
        got = lib.hils_decode_noalloc(*args, out=out, **kw)
        torch.cuda.synchronize()
        assert got[0] is out[0]
        for a, b, n in zip(got, ref, ("o", "lse", "topk_idx")):
            assert torch.equal(a, b), f"{wl.name}: {n} differs from the workspace path"
        od = H.hils_decode(t, wl.S, wl.K, wl.W, forced_topk=got[2].cpu().numpy())
        compare(f"{wl.name} o", got[0].cpu().double().numpy(), od["o"], wl.dtype)
        compare(f"{wl.name} lse", got[1].cpu().double().numpy(), od["lse"], wl.dtype,
                dict(max_abs=2e-3, mean_abs=2e-3))
