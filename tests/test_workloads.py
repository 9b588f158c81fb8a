"""The seeded input generators: N(0,1) draws with the normal law's tails,
and slabs that regenerate row by row (what lets the oracle rebuild only the
rows it checks at full size)."""
import math

import numpy as np
import torch
from scipy import stats

from workloads import (NORMAL_BITS, WORKLOADS, Workload, _counters, gen_slab, make_group_inputs,
                       make_inputs, normal_at, normal_table, slab_key)


def test_normal_table_is_the_quantile_function_at_bin_midpoints():
    tab = normal_table().double().numpy()
    n = 1 << NORMAL_BITS
    assert tab.shape == (n,)
    # antisymmetric, increasing, quantiles at (k + 1/2) / n
    np.testing.assert_allclose(tab, -tab[::-1], rtol=0, atol=1e-6)
    assert np.all(np.diff(tab) > 0)
    for k in (0, 1, 1000, n // 3, n - 1):
        np.testing.assert_allclose(stats.norm.cdf(tab[k]), (k + 0.5) / n, rtol=1e-5)
    np.testing.assert_allclose(tab[-1], stats.norm.isf(0.5 / n), rtol=1e-6)  # ~5.17


def test_normal_draws_have_normal_moments_and_tails():
    x = normal_at(slab_key(9, "q", 0, 0), _counters(1 << 22, "cpu")).double().numpy()
    n = x.size
    assert abs(x.mean()) < 5 / math.sqrt(n)
    assert abs(x.std() - 1.0) < 2e-3
    assert abs(stats.kurtosis(x)) < 0.02
    # mass beyond 3 and 4 standard deviations (Irwin-Hall(4) has none past 3.46)
    for z in (3.0, 4.0):
        p = 2 * stats.norm.sf(z)
        got = float((np.abs(x) > z).mean())
        assert abs(got - p) < 5 * math.sqrt(p / n) + 1e-7, (z, got, p)
    # a Kolmogorov-Smirnov test against N(0,1) on a sample
    assert stats.kstest(x[:200000], "norm").pvalue > 1e-3


def test_group_slabs_regenerate_bit_for_bit():
    wl = Workload("gen", seed=5, dtype="bf16", B=2, Hq=4, Hkv=2, d=64, N=512, S=64, K=4, W=128,
                  D=64, r=16, e_range=2.0, mode="train")
    t = make_inputs(wl)
    for b, g in ((0, 0), (1, 1)):
        tg = make_group_inputs(wl, b, g)
        assert torch.equal(tg["q"][0], t["q"][b, 2 * g:2 * g + 2])
        assert torch.equal(tg["k"][0, 0], t["k"][b, g])
        assert torch.equal(tg["dO"][0], t["dO"][b, 2 * g:2 * g + 2])
        assert torch.equal(tg["W_down"], t["W_down"][2 * g:2 * g + 2])
    rows = torch.tensor([3, 77, 400])
    part = gen_slab(wl, "k", 1, 0, None, rows=rows, row_len=64)
    assert torch.equal(part, t["k"][1, 0, rows])
