"""Benchmark: one step = route -> dispatch send -> dispatch recv -> combine on
one MI355X, over one batch of the DeepSeek-V3-shaped prefill share
(T=8192 tokens, H=7168, E=256, k=8, 32 virtual ranks x 8 local experts,
capacity T*k) unless --config names another workload.

Prints ONE JSON line: whole-step tokens/s, the per-kernel breakdown with
HIP-event durations on the launch stream, the HBM roofline of the dominant
kernel, and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config dsv3_prefill]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD public spec
SRC = os.path.join(ROOT, "combine_topk_route_amd", "csrc", "moe_route.hip")
TRAFFIC_WORKLOAD = "dsv3_prefill"   # the workload the committed counter runs measured
GRAPH_STEPS = 10                    # steps captured into one graph for graph_replay_multi
TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"traffic_{TRAFFIC_WORKLOAD}.txt")
VALU_FILE = os.path.join(ROOT, "profiles", f"valu_{TRAFFIC_WORKLOAD}.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", f"kernels_{TRAFFIC_WORKLOAD}.md")
CEILING_FILE = os.path.join(ROOT, "profiles", "hbm_ceiling.md")
# Where the timed launches find their inputs.
CACHE_STATE = {
    "step": ("device memory; steps back to back, so x (read once per step) stays in the "
             "256 MiB Infinity Cache from one step to the next, while y, buf and out stream "
             "through HBM"),
    "warm": "steady state: launches back to back, x cache-resident from the previous step",
    "cold": "every cache flushed before each launch (1 GiB read sweep): all inputs from HBM",
}
# VALU issue peak: 256 CUs x 4 SIMDs x 2.4 GHz, a wave64 instruction taking 4
# cycles on a 16-lane SIMD (packed fp32 is off): wave-instructions per second.
VALU_PEAK = 256 * 4 * 2.4e9 / 4


def algorithmic_bytes(cfg) -> dict:
    """Bytes each entry point must move: every row read or written once."""
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    P = T * k
    return {
        "route": 4 * T * E + 8 * P,
        "dispatch_send": 4 * P + 8 * P + 4 * E + 4 * (E + 1) + 4 * (R + 1),
        "dispatch_recv": 2 * T * H + 2 * P * H + 4 * P,
        "combine": 2 * P * H + 2 * T * H + 8 * P,
    }


def source_hash() -> str:
    """Hash of the kernel source's code: comments and blank lines are
    dropped, so editing a comment does not mark the counter runs stale."""
    with open(SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def _committed_count(path: str, kernel: str, workload: str, section: str = "kernels"):
    """A per-launch figure from a committed rocprofv3 summary (its JSON line,
    `section` of it), or None when there is none for this workload or the
    kernel source changed since the profile was taken."""
    if workload != TRAFFIC_WORKLOAD:
        return None
    try:
        with open(path) as f:
            rec = json.loads(f.read().split("JSON:", 1)[1].strip().splitlines()[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash():
        return None
    return rec.get(section, {}).get(kernel)


def measured_traffic(kernel: str, workload: str, cold: bool = False):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE runs
    (the launches after the cache flush when `cold`)."""
    return _committed_count(TRAFFIC_FILE, kernel, workload,
                            "kernels_cold" if cold else "kernels")


def chip_ceilings():
    """The chip's practical HBM rates from the committed probes.py
    hbm_ceiling summary (TB/s: streaming read / write / copy, and reads and
    writes of 1-16 KiB pieces in random order), or None without it."""
    try:
        with open(CEILING_FILE) as f:
            return json.loads(f.read().split("JSON:", 1)[1].strip().splitlines()[0])
    except (OSError, IndexError, ValueError):
        return None


def ceiling_bound(kernel: str, leg: str, cfg, ceil) -> dict:
    """A row kernel's time if its reads and its writes each ran alone, one
    after the other, at the chip's ceiling for their pattern, and the
    fraction of the 8 TB/s peak that gives on its algorithmic bytes.  recv
    reads each token row once, in order (streaming read; from the Infinity
    Cache when warm, so not counted), and writes 2 KiB pieces of the k
    destination rows at the expert segments (random-order writes).  Combine
    gathers its k expert rows (random-order reads) and writes each output row
    once, in order (streaming write).  The random-order figure stands for
    routing spread over many experts; a skewed routing writes more of its
    rows in order and can beat it (frac_of_bound above 1)."""
    T, H, P = cfg.T, cfg.H, cfg.P
    if kernel == "dispatch_recv":
        reads, writes = (2 * T * H, ceil["read_TBps"]), (2 * P * H + 4 * P, ceil["random_write_TBps"])
        if leg == "warm":
            reads = (0, reads[1])
    else:
        reads, writes = (2 * P * H + 8 * P, ceil["random_read_TBps"]), (2 * T * H, ceil["write_TBps"])
    us = reads[0] / reads[1] / 1e6 + writes[0] / writes[1] / 1e6
    nbytes = dict(algorithmic_bytes(cfg))[kernel]
    return {"us": round(us, 2), "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def alu_roofline(kernel: str, us: float, workload: str):
    """Routing is bound by VALU issue: its committed SQ_INSTS_VALU count per
    launch, the time that takes at the issue peak, and that time as a share
    of the measured launch time (None without a current count)."""
    n = _committed_count(VALU_FILE, kernel, workload)
    if n is None:
        return None
    issue_us = n / VALU_PEAK * 1e6
    return {"bound": "alu", "valu_insts": n, "peak_winst_per_s": VALU_PEAK,
            "issue_us": round(issue_us, 2), "frac": round(issue_us / us, 4)}


def cpu_baseline(cfg_name: str, sample_tokens: int, seed: int) -> dict:
    import numpy as np  # noqa: F401

    import oracle
    import workloads

    wl = workloads.make(cfg_name, seed=seed, T=sample_tokens)
    cfg = wl.cfg
    t0 = time.perf_counter()
    idx, _, w32 = oracle.route_topk(wl.logits, cfg.k)
    t1 = time.perf_counter()
    counts = oracle.expert_counts(idx, cfg.E)
    oracle.expert_offsets(counts)
    pr, _ = oracle.dispatch_slots(idx, cfg.E)
    oracle.dispatch_rows(wl.x, pr, sample_tokens * cfg.k)
    t2 = time.perf_counter()
    oracle.combine(wl.y, pr, w32)
    t3 = time.perf_counter()
    dt = t3 - t0
    return {
        "value": sample_tokens / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"first {sample_tokens} of {cfg.T} tokens of {cfg_name} (same seed and "
                   f"distribution), route+dispatch+combine in numpy, {dt:.1f} s (route "
                   f"{t1 - t0:.1f} s, dispatch {t2 - t1:.1f} s, combine {t3 - t2:.1f} s), "
                   f"host has {os.cpu_count()} cpus, affinity {len(os.sched_getaffinity(0))}"),
    }


# Tokens of each workload the per-config oracle table times (a few seconds
# of numpy each on one core).
CPU_TABLE_TOKENS = {"tiny": 16, "mixtral": 2048, "dsv3_decode": 128, "dsv3_prefill": 1024,
                    "kimi_k2": 1024}


def cpu_table(seed: int) -> dict:
    """The oracle timed on every workload (a bounded prefix of each, stages
    timed separately), and Tiny also in brute-force mode: exhaustive k-subset
    search for routing and exact rational arithmetic for every fma of
    combine.  numpy runs these element-wise loops on one core."""
    import numpy as np

    import oracle
    import workloads

    rows = []
    for name, n in CPU_TABLE_TOKENS.items():
        wl = workloads.make(name, seed=seed, T=n)
        cfg = wl.cfg
        t0 = time.perf_counter()
        idx, _, w32 = oracle.route_topk(wl.logits, cfg.k)
        t1 = time.perf_counter()
        counts = oracle.expert_counts(idx, cfg.E)
        oracle.expert_offsets(counts)
        pr, _ = oracle.dispatch_slots(idx, cfg.E)
        oracle.dispatch_rows(wl.x, pr, n * cfg.k)
        t2 = time.perf_counter()
        oracle.combine(wl.y, pr, w32)
        t3 = time.perf_counter()
        nb = algorithmic_bytes(dataclass_replace_T(cfg, n))
        rows.append({"workload": name, "tokens": n, "of": cfg.T, "route_s": round(t1 - t0, 4),
                     "dispatch_s": round(t2 - t1, 4), "combine_s": round(t3 - t2, 4),
                     "tokens_per_s": round(n / (t3 - t0), 1),
                     "dispatch_combine_GBps": round(
                         (nb["dispatch_recv"] + nb["combine"]) / (t3 - t1) / 1e9, 3)})
        if name == "tiny":
            t0 = time.perf_counter()
            sets = oracle.route_topk_bruteforce(wl.logits, cfg.k)
            t1 = time.perf_counter()
            exact = oracle.combine_exact(wl.y, pr, w32)
            t2 = time.perf_counter()
            assert [tuple(sorted(r)) for r in idx.tolist()] == [tuple(s_) for s_ in sets]
            assert np.array_equal(exact, oracle.combine(wl.y, pr, w32))
            rows.append({"workload": "tiny (brute force)", "tokens": n, "of": cfg.T,
                         "route_s": round(t1 - t0, 4), "combine_s": round(t2 - t1, 4),
                         "tokens_per_s": round(n / (t2 - t0), 1),
                         "note": "exhaustive subset search; exact-rational fma chain; "
                                 "both agree with the vectorised oracle"})
    return {"cpu_oracle_table": rows, "cores": 1, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)), "seed": seed}


def dataclass_replace_T(cfg, T: int):
    import dataclasses

    return dataclasses.replace(cfg, T=T)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3_prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-overlap", action="store_true", help="skip the two-stream overlap timing")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing (keeps a kernel trace to warm launches only)")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the CPU oracle on every workload (host only) and exit")
    args = ap.parse_args()

    if args.cpu_table:
        print(json.dumps(cpu_table(args.seed)), flush=True)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import combine_topk_route_amd as m
    import workloads

    cfg = workloads.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.make(cfg, seed=args.seed)
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    P = T * k

    logits = torch.from_numpy(wl.logits).to(dev)
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.from_numpy(wl.y.view(np.int16)).view(torch.bfloat16).to(dev)
    del wl
    # One set of preallocated buffers (the allocation-free API a serving loop
    # uses); the per-entry-point breakdown below writes into the same tensors.
    bufs = m.MoeBuffers(T, H, E, k, R, device=dev, fp8=H % 128 == 0)
    idx, w = bufs.topk_idx, bufs.topk_w
    counts, offsets, rank_off = bufs.expert_counts, bufs.expert_offsets, bufs.rank_offsets
    pair_row, row_token = bufs.pair_row, bufs.row_token
    ws = bufs.workspace
    buf, out = bufs.buf, bufs.out
    stream = torch.cuda.current_stream()

    def step(ev=None, st=None):
        """route -> send -> recv -> combine.  Without events, route, send and
        recv go through the one moe_route_dispatch call (the same kernels,
        route and send in one launch for small batches) and combine through
        moe_combine, both by way of MoeBuffers; with events, each entry point
        is bracketed on its own."""
        st = stream if st is None else st
        if ev is None:
            _, tw, send, _ = bufs.route_dispatch(logits, x, stream=st)
            bufs.combine(y, send.pair_row, tw, stream=st)
            return
        ev[0].record(st)
        m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w, stream=st)
        ev[1].record(st)
        m.moe_dispatch_send(idx, E, R, expert_counts=counts, expert_offsets=offsets,
                            pair_row=pair_row, row_token=row_token, rank_offsets=rank_off,
                            workspace=ws, stream=st)
        ev[2].record(st)
        m.moe_dispatch_recv(x, pair_row, buf=buf, stream=st)
        ev[3].record(st)
        m.moe_combine(y, pair_row, w, out=out, stream=st)
        ev[4].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1 (the headline): K steps back to back, events only at
    # the two ends.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # Timed region 2: the same K steps with an event pair around every entry
    # point on the launch stream (per-kernel durations for the roofline).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()

    # Routing alone, back to back on the GPU: K launches captured into one
    # HIP graph and replayed once (an event pair per launch adds a few
    # microseconds of record overhead, the size of the kernel itself, and
    # eager launches from Python can leave the GPU waiting for the host).
    route_b2b_us = None
    if not args.no_graph:
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w, stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for _ in range(args.steps):
                m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w,
                                 stream=torch.cuda.current_stream())
        gr.replay()
        torch.cuda.synchronize()
        ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ra.record(stream)
        gr.replay()
        rb.record(stream)
        torch.cuda.synchronize()
        route_b2b_us = ra.elapsed_time(rb) * 1000.0 / args.steps
        del gr

    # Timed region 3: the step captured once into a HIP graph (no host-side
    # knowledge of routed counts is needed, so one graph serves any routing)
    # and replayed K times.
    graph_ms = graph10_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(st=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step(st=torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(args.steps):
            g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / args.steps
        # The same with GRAPH_STEPS steps in one graph, as a captured pass over
        # many layers would hold: the launch cost of a graph is per replay.
        g10 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g10):
            for _ in range(GRAPH_STEPS):
                step(st=torch.cuda.current_stream())
        g10.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // GRAPH_STEPS)
        ga.record(stream)
        for _ in range(reps):
            g10.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph10_ms = ga.elapsed_time(gb) / (reps * GRAPH_STEPS)
        del g, g10

    # Timed region 4 (cold caches): every entry point again, each launch
    # preceded by a read sweep over 1 GiB that evicts L2 and the Infinity
    # Cache (a read sweep leaves no dirty lines to write back during the
    # timed launch), plus send + recv as the single moe_dispatch call.
    cold_names = [] if args.no_cold else ["route", "dispatch_send", "dispatch_recv", "combine",
                                          "dispatch"]
    flush = torch.empty((1 << 28 if cold_names else 1,), dtype=torch.float32, device=dev).fill_(1.0)
    cold_calls = {
        "route": lambda: m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w, stream=stream),
        "dispatch_send": lambda: m.moe_dispatch_send(
            idx, E, R, expert_counts=counts, expert_offsets=offsets, pair_row=pair_row,
            row_token=row_token, rank_offsets=rank_off, workspace=ws, stream=stream),
        "dispatch_recv": lambda: m.moe_dispatch_recv(x, pair_row, buf=buf, stream=stream),
        "combine": lambda: m.moe_combine(y, pair_row, w, out=out, stream=stream),
        "dispatch": lambda: m.moe_dispatch(
            idx, x, E, R, buf=buf, expert_counts=counts, expert_offsets=offsets,
            pair_row=pair_row, row_token=row_token, rank_offsets=rank_off, workspace=ws,
            stream=stream),
    }
    cold_ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)] for n in cold_names}
    torch.cuda.synchronize()
    for i in range(args.steps):
        for n in cold_names:
            flush.amax()
            cold_ev[n][i][0].record(stream)
            cold_calls[n]()
            cold_ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    del flush

    # Block-scaled fp8 dispatch, the pages' own dispatch payload (codes and
    # one fp32 scale per 128 elements; combine stays 16-bit): the recv alone,
    # warm and after the cache sweep, and the whole step with it.
    fp8 = None
    if H % 128 == 0:
        buf_q, buf_s = bufs.buf_q, bufs.buf_scale
        fp8_call = lambda: m.moe_dispatch_recv_fp8(x, pair_row, buf_q=buf_q, buf_scale=buf_s,
                                                   stream=stream)
        fp8_call()
        flush = (torch.empty((1 << 28,), dtype=torch.float32, device=dev).fill_(1.0)
                 if not args.no_cold else None)
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps if flush is not None else 0)]
        torch.cuda.synchronize()
        for a_, b_ in fev:
            a_.record(stream)
            fp8_call()
            b_.record(stream)
        for a_, b_ in cev:
            flush.amax()
            a_.record(stream)
            fp8_call()
            b_.record(stream)
        torch.cuda.synchronize()
        del flush
        fb = 2 * T * H + P * H + 4 * P * (H // 128) + 4 * P

        def leg(evl):
            us_ = 1000.0 * float(np.mean([a_.elapsed_time(b_) for a_, b_ in evl]))
            return {"us_mean": round(us_, 2), "GBps": round(fb / (us_ * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(fb / (us_ * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}

        fp8 = dict(leg(fev), bytes=fb, traffic=measured_traffic("fp8_dispatch_recv", cfg.name),
                   speedup_vs_bf16_recv=None, cold=leg(cev) if cev else None)

        def step_fp8():
            _, tw, send, _, _ = bufs.route_dispatch_fp8(logits, x, stream=stream)
            bufs.combine(y, send.pair_row, tw, stream=stream)

        for _ in range(max(1, args.warmup)):
            step_fp8()
        torch.cuda.synchronize()
        sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sa.record(stream)
        for _ in range(args.steps):
            step_fp8()
        sb.record(stream)
        torch.cuda.synchronize()
        ms_fp8 = sa.elapsed_time(sb) / args.steps
        fp8["step"] = {"ms_per_step": round(ms_fp8, 4),
                       "tokens_per_s": round(T / (ms_fp8 * 1e-3), 1),
                       "what": "moe_route_dispatch_fp8 + moe_combine (bf16 y), back to back"}
        # the headline's routing tables again, for anything timed after this
        m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w, stream=stream)
        m.moe_dispatch_send(idx, E, R, expert_counts=counts, expert_offsets=offsets,
                            pair_row=pair_row, row_token=row_token, rank_offsets=rank_off,
                            workspace=ws, stream=stream)
        torch.cuda.synchronize()

    # Group-limited routing (DeepSeek-V3's grouping: 8 groups of E/8 experts,
    # the 4 best kept) on the same logits, timed on its own like fp8 above.
    route_grouped = None
    n_group, topk_group = 8, 4
    if E % n_group == 0 and k <= topk_group * (E // n_group):
        m.moe_route_topk_grouped(logits, k, n_group, topk_group, topk_idx=idx, topk_w=w,
                                 stream=stream)
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a_, b_ in gev:
            a_.record(stream)
            m.moe_route_topk_grouped(logits, k, n_group, topk_group, topk_idx=idx, topk_w=w,
                                     stream=stream)
            b_.record(stream)
        torch.cuda.synchronize()
        us = 1000.0 * float(np.mean([a_.elapsed_time(b_) for a_, b_ in gev]))
        gb = algorithmic_bytes(cfg)["route"]
        route_grouped = {"n_group": n_group, "topk_group": topk_group, "us_mean": round(us, 2),
                         "bytes": gb, "GBps": round(gb / (us * 1e-6) / 1e9, 1),
                         "frac_of_peak": round(gb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "alu": None}
        g_trace = _committed_count(TRACE_FILE, "route_grouped", cfg.name)
        if g_trace is not None:
            a_ = alu_roofline("route_grouped", g_trace, cfg.name)
            route_grouped["alu"] = None if a_ is None else dict(a_, us_trace=g_trace)
        # the headline's routing outputs again, for anything timed after this
        m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w, stream=stream)
        torch.cuda.synchronize()

    # Overlap: dispatch (send + recv) on the launch stream while a stand-in
    # shared-expert GEMM, x[T,H] @ W[H, 2048] in bf16, runs on a second
    # stream (both at the default priority).  hidden = (t_dispatch + t_gemm
    # - t_both) / min(t_dispatch, t_gemm).
    overlap = None
    if not args.no_overlap:
        wsh = torch.randn((H, 2048), device=dev, dtype=torch.float32).to(torch.bfloat16)
        gout = torch.empty((T, 2048), dtype=torch.bfloat16, device=dev)
        other = torch.cuda.Stream()

        def disp(st):
            m.moe_dispatch_send(idx, E, R, expert_counts=counts, expert_offsets=offsets,
                                pair_row=pair_row, row_token=row_token, rank_offsets=rank_off,
                                workspace=ws, stream=st)
            m.moe_dispatch_recv(x, pair_row, buf=buf, stream=st)

        def gemm():
            torch.matmul(x, wsh, out=gout)

        def timed(fn, reps=10):
            fn()
            torch.cuda.synchronize()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(reps):
                fn()
            b_.record(stream)
            torch.cuda.synchronize()
            return a_.elapsed_time(b_) * 1000.0 / reps

        def both():
            other.wait_stream(stream)
            with torch.cuda.stream(other):
                gemm()
            disp(stream)
            stream.wait_stream(other)

        t_d = timed(lambda: disp(stream))
        t_g = timed(gemm)
        t_b = timed(both)
        overlap = {"dispatch_us": round(t_d, 1), "shared_gemm_us": round(t_g, 1),
                   "concurrent_us": round(t_b, 1),
                   "hidden_frac": round((t_d + t_g - t_b) / min(t_d, t_g), 3),
                   "gemm": f"[{T},{H}] x [{H},2048] bf16 (stand-in shared expert)"}
        del wsh, gout

    names = ["route", "dispatch_send", "dispatch_recv", "combine"]
    per = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n].append(e[j].elapsed_time(e[j + 1]))
    nbytes = algorithmic_bytes(cfg)
    kernels = {}
    for n in names:
        us = 1000.0 * float(np.mean(per[n]))
        gbps = nbytes[n] / (us * 1e-6) / 1e9
        kernels[n] = {"us_mean": round(us, 2), "us_median": round(1000 * float(np.median(per[n])), 2),
                      "us_p10": round(1000 * float(np.percentile(per[n], 10)), 2),
                      "us_p90": round(1000 * float(np.percentile(per[n], 90)), 2),
                      "bytes": nbytes[n], "GBps": round(gbps, 1),
                      "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    # Routing's ALU roofline: VALU issue time over the kernel's own duration,
    # the committed kernel trace's average for the same code (an event pair
    # per launch adds record overhead of the kernel's own size, and
    # back-to-back graph replay a launch gap of about a microsecond per
    # kernel; the live back-to-back figure is reported beside it).  The
    # counting kernel of the headline step runs inside moe_route_dispatch,
    # where no event can bracket it.
    if route_b2b_us is not None:
        kernels["route"]["us_back_to_back"] = round(route_b2b_us, 2)
    for key, name in (("alu", "route"), ("alu_counting", "route_counting")):
        trace_us = _committed_count(TRACE_FILE, name, cfg.name)
        if trace_us is not None:
            a_ = alu_roofline(name, trace_us, cfg.name)
            if a_ is not None:
                kernels["route"][key] = dict(a_, us_trace=trace_us)
                if name == "route" and route_b2b_us is not None:
                    kernels["route"][key]["frac_back_to_back"] = round(
                        a_["issue_us"] / route_b2b_us, 4)
    nbytes_cold = dict(nbytes, dispatch=nbytes["dispatch_send"] + nbytes["dispatch_recv"])
    kernels_cold = {}
    for n in cold_names:
        d = [a_.elapsed_time(b_) for a_, b_ in cold_ev[n]]
        med = 1000.0 * float(np.median(d))
        mean = 1000.0 * float(np.mean(d))
        kernels_cold[n] = {"us_mean": round(mean, 2), "us_median": round(med, 2),
                           "us_p10": round(1000 * float(np.percentile(d, 10)), 2),
                           "us_p90": round(1000 * float(np.percentile(d, 90)), 2),
                           "GBps": round(nbytes_cold[n] / (mean * 1e-6) / 1e9, 1),
                           "frac_of_peak": round(nbytes_cold[n] / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    # The row kernels' roofline, warm (back-to-back steps: x stays in the
    # Infinity Cache from one step to the next) and cold (every cache flushed
    # before the launch).  The cold protocol is the one of record when it
    # ran; the dominant kernel is the slower row kernel under it.
    row_roof = {}
    for n in ("dispatch_recv", "combine"):
        row_roof[n] = {"bytes": nbytes[n],
                       "warm": {"us_mean": kernels[n]["us_mean"], "GBps": kernels[n]["GBps"],
                                "frac": kernels[n]["frac_of_peak"]}}
        if n in kernels_cold:
            row_roof[n]["cold"] = {"us_mean": kernels_cold[n]["us_mean"],
                                   "GBps": kernels_cold[n]["GBps"],
                                   "frac": kernels_cold[n]["frac_of_peak"]}
    ceil = chip_ceilings()
    if ceil is not None:
        for n in row_roof:
            for lg in ("warm", "cold"):
                if lg in row_roof[n]:
                    b = ceiling_bound(n, lg, cfg, ceil)
                    row_roof[n][lg]["chip_bound"] = dict(
                        b, frac_of_bound=round(row_roof[n][lg]["frac"] / b["frac"], 4))
    leg = "cold" if kernels_cold else "warm"
    dom = max(["dispatch_recv", "combine"], key=lambda n: row_roof[n][leg]["us_mean"])
    if fp8 is not None:
        fp8["speedup_vs_bf16_recv"] = round(kernels["dispatch_recv"]["us_mean"] / fp8["us_mean"], 3)
    step_bytes = sum(nbytes.values())
    tokens_per_s = T * args.steps / (total_ms * 1e-3)

    # A plain 1 GiB device copy: the practical bandwidth ceiling, and the
    # reference kernel of known size for scaling FETCH_SIZE / WRITE_SIZE.
    src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    traffic = measured_traffic(dom, cfg.name, cold=leg == "cold")
    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "virtual_ranks": R,
                   "local_experts": cfg.L, "capacity": P, "seed": args.seed,
                   "step": "route+dispatch_send+dispatch_recv+combine",
                   "accumulate": "fp32", "inputs": CACHE_STATE["step"]},
        "hbm_GBps_step": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_frac_step": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {
            "kernel": dom,
            "cache": CACHE_STATE[leg],
            "bound": "hbm",
            "achieved": row_roof[dom][leg]["GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": row_roof[dom][leg]["frac"],
            "traffic": traffic,
            "chip_ceilings_TBps": ceil,
            "chip_bound": row_roof[dom][leg].get("chip_bound"),
            "row_kernels": row_roof,
        },
        "kernels": kernels,
        "kernels_cold": kernels_cold or None,
        "fp8_dispatch_recv": fp8,
        "route_grouped": route_grouped,
        "overlap": overlap,
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 4),
            "tokens_per_s": round(T / (graph_ms * 1e-3), 1)},
        "graph_replay_multi": None if graph10_ms is None else {
            "steps_per_graph": GRAPH_STEPS,
            "ms_per_step": round(graph10_ms, 4),
            "tokens_per_s": round(T / (graph10_ms * 1e-3), 1)},
        "copy_1GiB_GBps": round(copy_gbps, 1),
        "host_wall_s": round(t_host, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg.name, min(args.cpu_sample_tokens, T), args.seed)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
