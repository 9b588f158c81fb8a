"""Host-side logic of bench.py (no GPU): the algorithmic work it divides by,
the oracle baseline's process fan-out, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def brute_counts(wl):
    """Window tokens, selected-chunk tokens and distant chunks summed over
    positions, by walking every position and chunk (causal: chunk c is
    distant for position i when its newest token c*S + S - 1 <= i - W)."""
    win = chk = dist = 0
    for i in range(wl.N):
        nd = sum(1 for c in range(wl.N // wl.S) if c * wl.S + wl.S - 1 <= i - wl.W)
        dist += nd
        chk += min(wl.K, nd) * wl.S
        win += i + 1 - nd * wl.S
    return win, chk, dist


@pytest.mark.parametrize("kw", [dict(), dict(N=1000, W=100, K=3), dict(N=700, W=64, S=64, K=16),
                                dict(N=64, W=128)])
def test_algorithmic_work_matches_brute_force(kw):
    wl = WORKLOADS["tiny"].with_(**kw)
    win, chk, dist = brute_counts(wl)
    fw, fc = bench.fwd_algorithmic_flops(wl)
    rows = wl.B * wl.Hq
    assert fw == rows * 4 * wl.d * win
    assert fc == rows * 4 * wl.d * chk
    assert bench.route_algorithmic_flops(wl) == rows * 2 * wl.d * dist


def test_config_flops_are_the_stated_totals():
    """345M prefill: 1.903e11 attention flops, 3.744e9 routing flops; the
    131072-token GQA prefill: 4.430e12 and 1.082e12."""
    fw, fc = bench.fwd_algorithmic_flops(WORKLOADS["prefill_345m"])
    assert round((fw + fc) / 1e8) == 1903
    assert round(bench.route_algorithmic_flops(WORKLOADS["prefill_345m"]) / 1e6) == 3744
    fw, fc = bench.fwd_algorithmic_flops(WORKLOADS["prefill_1p4b"])
    assert round((fw + fc) / 1e9) == 4430
    assert round(bench.route_algorithmic_flops(WORKLOADS["prefill_1p4b"]) / 1e9) == 1082


def test_deal_covers_every_task_once():
    tasks = list(range(37))
    for nw in (1, 5, 16, 64):
        parts = bench._deal(tasks, nw)
        assert len(parts) == min(nw, len(tasks))
        assert all(parts)
        assert sorted(x for p in parts for x in p) == tasks


def test_traffic_is_null_without_a_matching_summary():
    assert bench.recorded_traffic("window", "no_such_workload") is None


def test_oracle_workers_run_in_parallel_processes():
    """Two forked single-threaded workers over a few rows of the tiny
    workload: every unit is counted, the wall time is positive."""
    wl = WORKLOADS["tiny"]
    tasks = [[(wl.name, 0, 0, [2047, 1500])], [(wl.name, 0, 0, [1024, 700, 300])]]
    units, wall, used = bench.run_oracle_workers("prefill", tasks, timeout_s=300)
    assert (units, used) == (5, 2) and wall > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
