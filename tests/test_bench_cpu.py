"""bench.py's host-side pieces (no GPU): the algorithmic byte counts the
roofline uses, the counter-traffic and VALU-count lookups, the bound from
the chip's measured ceilings, and the one-GPU guard."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_at_dsv3_prefill():
    cfg = workloads.CONFIGS["dsv3_prefill"]
    b = bench.algorithmic_bytes(cfg)
    T, H, k = cfg.T, cfg.H, cfg.k
    # per token: 2H(k+1) bytes of rows, plus 4 (recv) or 8 (combine) bytes per pair
    assert b["dispatch_recv"] == T * (2 * H * (k + 1) + 4 * k) == 1_057_226_752
    assert b["combine"] == T * (2 * H * (k + 1) + 8 * k) == 1_057_488_896
    assert b["route"] == T * (4 * cfg.E + 8 * k)


def test_traffic_is_only_reported_for_the_measured_workload_and_source():
    assert bench.measured_traffic("combine", "kimi_k2") is None
    got = bench.measured_traffic("combine", bench.TRAFFIC_WORKLOAD)
    if got is not None:  # the committed counters match the current kernel source
        alg = bench.algorithmic_bytes(workloads.CONFIGS[bench.TRAFFIC_WORKLOAD])["combine"]
        assert 1.0 <= got / alg < 1.05


def test_alu_roofline_uses_the_committed_valu_count():
    assert bench.alu_roofline("route", 10.0, "kimi_k2") is None
    got = bench.alu_roofline("route", 10.0, bench.TRAFFIC_WORKLOAD)
    if got is not None:  # the committed counters match the current kernel source
        # 256 CUs x 4 SIMDs x 2.4 GHz / 4 cycles per wave64 instruction
        assert got["peak_winst_per_s"] == 614.4e9
        assert abs(got["issue_us"] - got["valu_insts"] / 614.4e3) < 0.01
        assert abs(got["frac"] - got["valu_insts"] / 614.4e3 / 10.0) < 1e-4
        cfg = workloads.CONFIGS[bench.TRAFFIC_WORKLOAD]
        # the routing kernel issues a few hundred VALU instructions per token
        assert 100 < got["valu_insts"] / cfg.T < 2000


def test_chip_bound_from_the_committed_ceilings():
    """Each row kernel's bound: its reads and writes one after the other at
    the chip's measured ceilings for their pattern; recv's warm bound leaves
    out the cache-resident x, so it is the tighter of recv's two."""
    c = bench.chip_ceilings()
    assert c is not None and set(c) >= {"read_TBps", "write_TBps", "random_write_TBps",
                                        "random_read_TBps"}
    assert c["random_write_TBps"] < c["write_TBps"] < c["read_TBps"] < 8.0
    cfg = workloads.CONFIGS["dsv3_prefill"]
    T, H, P = cfg.T, cfg.H, cfg.P
    warm = bench.ceiling_bound("dispatch_recv", "warm", cfg, c)
    cold = bench.ceiling_bound("dispatch_recv", "cold", cfg, c)
    assert abs(warm["us"] - (2 * P * H + 4 * P) / c["random_write_TBps"] / 1e6) < 0.01
    assert abs(cold["us"] - warm["us"] - 2 * T * H / c["read_TBps"] / 1e6) < 0.02
    assert cold["frac"] < warm["frac"] < 1.0
    comb = bench.ceiling_bound("combine", "cold", cfg, c)
    assert comb == bench.ceiling_bound("combine", "warm", cfg, c)
    want = (2 * P * H + 8 * P) / c["random_read_TBps"] / 1e6 + 2 * T * H / c["write_TBps"] / 1e6
    assert abs(comb["us"] - want) < 0.01 and comb["frac"] < 1.0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
