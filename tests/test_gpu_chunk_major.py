"""The chunk-major forward strategy (each selected chunk loaded once for all
the rows that chose it, per-chunk outputs fused with the window's in a
second pass) against the fp64 oracle: every row of small cases across
dtypes, GQA groups, head dims, Q-Cal and ragged tails; degenerate lengths;
extreme token scores; and the same selection and outputs as the packed-union
strategy. Long sequences take this strategy by default; their full-size runs
are in test_gpu_long.py."""
import numpy as np
import pytest
import torch

from workloads import Workload, make_inputs
from tests.hils_testutil import fwd_parity, say, to_dev

pytestmark = pytest.mark.gpu


def L():
    import learnable_chunk_sparse_amd as lib
    return lib


def run(wl, td, strategy):
    out = L().hils_attn_fwd(td["q"], td["k"], td["v"], td["kL"], td["e"], wl.S, wl.K, wl.W,
                            h=td.get("h"), W_down=td.get("W_down"), W_up=td.get("W_up"),
                            strategy=strategy)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, dtype, B, Hq, Hkv, d, N, K, W, D, r, e_shift
    ("cm_mha_d64_qcal", "bf16", 2, 2, 2, 64, 1000, 4, 128, 64, 32, 0.0),
    ("cm_mha_d64_chunkdom", "bf16", 1, 2, 2, 64, 1100, 6, 128, 0, 0, 8.0),
    ("cm_gqa2_d128", "bf16", 1, 4, 2, 128, 900, 5, 192, 96, 16, 3.0),
    ("cm_gqa4_d128_qcal_k32", "bf16", 1, 8, 2, 128, 2500, 32, 256, 128, 32, 1.0),
    ("cm_gqa4_d64_r64", "bf16", 1, 4, 1, 64, 777, 3, 64, 64, 64, 2.0),
    ("cm_gqa2_d64_k7_tail", "bf16", 2, 4, 2, 64, 1999, 7, 128, 0, 0, 2.0),
    ("cm_fp32_d64", "fp32", 1, 2, 1, 64, 700, 4, 128, 0, 0, 4.0),
    ("cm_fp32_d64_qcal_gqa2", "fp32", 1, 4, 2, 64, 1520, 3, 64, 64, 32, 1.0),
    ("cm_fp32_d128_gqa4", "fp32", 1, 8, 2, 128, 1450, 5, 64, 0, 0, 2.0),
    ("cm_mha_d128_k1", "bf16", 1, 2, 2, 128, 3000, 1, 512, 0, 0, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_major_all_rows(case):
    name, dt, B, Hq, Hkv, d, N, K, W, D, r, sh = case
    wl = Workload(name, seed=51, dtype=dt, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, S=64, K=K, W=W, D=D, r=r,
                  e_range=2.0, e_shift=sh)
    say(f"case {name}")
    t = make_inputs(wl)
    td = to_dev(t)
    lib = L()
    out = run(wl, td, lib.FWD_CHUNK_MAJOR)
    fwd_parity(t, out, wl.S, wl.K, wl.W, dt, label=name)
    # the same selection, and outputs within the bar of the union strategy's
    ou, lu, iu = run(wl, td, lib.FWD_UNION)
    assert torch.equal(out[2], iu)
    tol = 2e-2 if dt == "bf16" else 1e-5
    assert float((out[0].float() - ou.float()).abs().max()) <= tol
    assert float((out[1] - lu).abs().max()) <= (2e-3 if dt == "bf16" else 1e-5)


@pytest.mark.parametrize("N", [1, 50, 64, 100, 191, 700])
def test_chunk_major_short_sequences(N):
    """No complete chunk (N < 64), no distant chunk (N < W + S), few distant chunks."""
    wl = Workload(f"cm_short{N}", seed=53, dtype="bf16", B=2, Hq=4, Hkv=2, d=64, N=N, S=64, K=4,
                  W=128, D=64, r=32, e_range=2.0)
    say(f"case chunk-major short N={N}")
    t = make_inputs(wl)
    out = run(wl, to_dev(t), L().FWD_CHUNK_MAJOR)
    fwd_parity(t, out, wl.S, wl.K, wl.W, "bf16", label=f"cm_short{N}")


def test_chunk_major_extreme_token_scores():
    """Chunk keys scaled up far above the window's scores and window keys far
    above the chunks': each chunk's softmax takes its own maximum."""
    wl = Workload("cm_extreme", seed=54, dtype="bf16", B=1, Hq=4, Hkv=2, d=64, N=1100, S=64, K=6,
                  W=128, D=0, r=0, e_range=2.0, e_shift=6.0)
    say("case chunk-major extreme token scores")
    t = make_inputs(wl)
    k = t["k"].float()
    k[:, :, 128:384] *= 45.0
    k[:, :, 1004:] *= 45.0
    t["k"] = k.to(torch.bfloat16)
    out = run(wl, to_dev(t), L().FWD_CHUNK_MAJOR)
    fwd_parity(t, out, wl.S, wl.K, wl.W, "bf16", label="cm_extreme")


def test_chunk_major_is_deterministic():
    """Two calls give identical bits (the inverse index is a stable sort)."""
    wl = Workload("cm_det", seed=55, dtype="bf16", B=1, Hq=8, Hkv=2, d=128, N=3000, S=64, K=8,
                  W=256, D=0, r=0, e_range=2.0)
    t = make_inputs(wl)
    td = to_dev(t)
    a = run(wl, td, L().FWD_CHUNK_MAJOR)
    b = run(wl, td, L().FWD_CHUNK_MAJOR)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
