"""Long-context prefill at full size: the paper's 512K-token measurement
setup (345M shape: 16 heads, d = 64, batch 1, chunk 64, top-32, a 512-token
window; one planted needle chunk per 16384-token segment), run through the
default strategy (chunk-major at this length) and checked against the fp64
oracle on sampled rows of two heads, every selection of those rows
included."""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_inputs, needle_rows_for_oracle
from tests.hils_testutil import say
from tests.test_gpu_fwd import group_parity, sample_rows

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def test_fwd_prefill_512k_full_size_sampled():
    wl = WORKLOADS["prefill_345m_512k"]
    say("case prefill_345m_512k full size: generating inputs on the GPU")
    t = make_inputs(wl, device="cuda")
    say("prefill_345m_512k: forward")
    out = L().hils_attn_fwd(t["q"], t["k"], t["v"], t["kL"], t["e"], wl.S, wl.K, wl.W, h=t["h"],
                            W_down=t["W_down"], W_up=t["W_up"])
    torch.cuda.synchronize()
    out = tuple(x.cpu() for x in out)
    idx = out[2]
    # every row far enough from the start holds K distinct chunks, all distant
    N, S, W = wl.N, wl.S, wl.W
    last = idx[0, :, N - 1]
    assert bool((last >= 0).all()) and int(last.max()) < (N - 1 - W + 1) // S
    for g in (0, 9):
        assert len(set(last[g].tolist())) == wl.K
    say(f"prefill_345m_512k: {len(needle_rows_for_oracle(wl, 0, 0))} needle chunks per head planted")
    del t["h"]
    group_parity(wl, t, out, [(0, 0), (0, 9)], sample_rows(wl, 40), "prefill_345m_512k")
