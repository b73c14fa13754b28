"""Measurements behind the shapes of the row kernels, on one MI355X.

    python probes.py recv_slices [--config dsv3_prefill] [--reps 20]
    python probes.py skew [--reps 20]
    python probes.py write_fronts [--config dsv3_prefill] [--launches 3]
    python probes.py cu_scaling [--config dsv3_prefill] [--reps 20]
    python probes.py overlap_masked [--config dsv3_prefill] [--reps 20]
    python probes.py store_policy [--config dsv3_prefill] [--reps 20]
    python probes.py hbm_ceiling [--reps 20]
    python probes.py combine_store [--reps 20]

Each prints one JSON line (write_fronts prints it after its launches, which a
rocprofv3 --pmc run records per dispatch).

* recv_slices: the recv kernel with 1, 2 and 4 slices (1 KiB column pieces of
  a token row) per wave, warm (right after a combine, as in back-to-back
  steps, where x stays in the Infinity Cache) and cold (after a 1 GiB read
  sweep that evicts every cache).  Slice counts other than the library's
  come from libraries built from the same source with MOE_RECV_SLICES
  (``python -m combine_topk_route_amd.build`` builds the product; this script
  builds the variants under _build/ when they are missing).
* skew: the same at the DSv3 prefill shape over Zipf-skewed routings, with
  the effective number of experts n_eff = P^2 / sum_e count_e^2.
* write_fronts: recv and combine on the workload's routing and on adjacent
  rows (pair_row[t, j] = t*k + j: each token's k destinations side by side),
  `launches` times each, in that order: recv real, recv adjacent, combine
  real, combine adjacent.
* cu_scaling: recv on streams restricted to n of the chip's CUs
  (hipExtStreamCreateWithCUMask), n = 32 .. all, CUs taken evenly over the
  chip or the first n.
* store_policy: the recv kernel with its stores as buffer stores under each
  cache policy (plain write-back, sc0, nt, sc1, nt sc1; MOE_RECV_STORE)
  against the library's global non-temporal stores, warm and cold.
* combine_store: moe_combine as built (sc1 output stores above 256 MiB of
  combine bytes, write-back below) against builds that force either form
  (MOE_COMBINE_SC1_MIN_BYTES), on every workload, warm and cold.
* hbm_ceiling: the chip's practical HBM rates for plain streaming kernels
  (read, write and copy over 4 GiB at several grid sizes), and chunk writes
  and reads of 1-16 KiB in order against a random order: the ceilings the
  row kernels are held against besides the 8 TB/s peak.
* overlap_masked: dispatch beside the stand-in shared-expert GEMM, back to
  back, on two unmasked streams, and with the CUs split between two masked
  streams.

All inputs are the seeded synthetic workloads of ``workloads``.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LIB_SLICES = 2  # the library's slices per recv wave (MOE_RECV_SLICES default)


def _setup(name, seed=0, zipf_s="config"):
    import numpy as np
    import torch

    import combine_topk_route_amd as m
    import workloads

    cfg = workloads.CONFIGS[name]
    if zipf_s != "config":
        cfg = dataclasses.replace(cfg, zipf_s=zipf_s, hot_bias=None, hot_rank=None)
    wl = workloads.make(cfg, seed=seed)
    dev = torch.device("cuda:0")
    d = dict(cfg=cfg,
             logits=torch.from_numpy(wl.logits).to(dev),
             x=torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(dev),
             y=torch.from_numpy(wl.y.view(np.int16)).view(torch.bfloat16).to(dev))
    del wl
    d["idx"], d["w"] = m.moe_route_topk(d["logits"], cfg.k)
    d["send"] = m.moe_dispatch_send(d["idx"], cfg.E, cfg.R)
    d["buf"] = torch.empty((cfg.P, cfg.H), dtype=torch.bfloat16, device=dev)
    d["out"] = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    c = d["send"].expert_counts.double()
    d["n_eff"] = float(cfg.P * cfg.P / (c * c).sum())
    d["active_experts"] = int((c > 0).sum())
    return d


def _recv_variant(name=None, defines=()):
    """C entry moe_dispatch_recv of the library (name None) or of the
    measurement build `name` with `defines`."""
    import combine_topk_route_amd as m
    from combine_topk_route_amd import build as b

    if name is None:
        return m._lib.load().moe_dispatch_recv
    path = b.variant_path(name)
    if not os.path.exists(path):
        b.build_variant(name, defines)
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.moe_dispatch_recv.argtypes = [vp, vp, i64, i32, i32, vp, i64, vp]
    lib.moe_dispatch_recv.restype = ctypes.c_int
    return lib.moe_dispatch_recv


def _slice_variant(slices):
    if slices == LIB_SLICES:
        return None, ()
    return f"recv_slices_{slices}", (f"MOE_RECV_SLICES={slices}",)


# Store forms of the recv kernel: cache-policy words of a buffer store
# (sc0 = 1, nt = 2, sc1 = 16); the library uses a global non-temporal store.
STORE_FORMS = {"plain": 0, "sc0": 1, "nt": 2, "sc1": 16, "nt sc1": 18}


def _store_variant(form):
    cpol = STORE_FORMS[form]
    return f"recv_store_{cpol}", (f"MOE_RECV_STORE={cpol}",)


class _Timer:
    def __init__(self, reps, rounds=3):
        import torch

        self.reps, self.rounds = reps, rounds
        self.stream = torch.cuda.current_stream()
        self.flush = torch.empty((1 << 28,), dtype=torch.float32,
                                 device="cuda").fill_(1.0)  # 1 GiB

    def median_us(self, fn, pre):
        """Median over rounds of the median of `reps` launches, each after `pre`."""
        import numpy as np
        import torch

        meds = []
        for _ in range(self.rounds):
            ev = []
            for _ in range(self.reps):
                pre()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(self.stream)
                fn()
                b.record(self.stream)
                ev.append((a, b))
            torch.cuda.synchronize()
            meds.append(float(np.median([a.elapsed_time(b) * 1000.0 for a, b in ev])))
        return float(np.median(meds))

    def cold(self):
        self.flush.amax()


def _recv_bytes(cfg):
    return 2 * cfg.T * cfg.H + 2 * cfg.P * cfg.H + 4 * cfg.P


def _variant_rows(d, timer, variants):
    """variants: (label, name, defines) -> warm/cold rows, each buffer
    checked bit for bit against the library's."""
    import torch

    import combine_topk_route_amd as m

    cfg = d["cfg"]
    st = timer.stream.cuda_stream
    ref = m.moe_dispatch_recv(d["x"], d["send"].pair_row)
    comb = lambda: m.moe_combine(d["y"], d["send"].pair_row, d["w"], out=d["out"],
                                 stream=timer.stream)
    rows = []
    for label, name, defines in variants:
        fn_c = _recv_variant(name, defines)
        call = lambda: fn_c(d["x"].data_ptr(), d["send"].pair_row.data_ptr(), cfg.T, cfg.H,
                            cfg.k, d["buf"].data_ptr(), cfg.P, st)
        d["buf"].zero_()
        rc = call()
        torch.cuda.synchronize()
        same = rc == 0 and torch.equal(d["buf"].view(torch.int16), ref.view(torch.int16))
        warm = timer.median_us(call, comb)
        cold = timer.median_us(call, timer.cold)
        nb = _recv_bytes(cfg)
        rows.append({"variant": label, "library": name is None, "bit_exact": bool(same),
                     "warm_us": round(warm, 1), "cold_us": round(cold, 1),
                     "warm_frac": round(nb / warm / 1e3 / 8000.0, 4),
                     "cold_frac": round(nb / cold / 1e3 / 8000.0, 4)})
        print(f"[probe] {cfg.name} {label}: warm {warm:.1f} us cold {cold:.1f} us",
              file=sys.stderr, flush=True)
    del ref
    return rows


def _slices_rows(d, timer, slices_list):
    rows = _variant_rows(d, timer, [(u, *_slice_variant(u)) for u in slices_list])
    for r in rows:
        r["slices"] = r.pop("variant")
    return rows


def probe_recv_slices(args):
    timer = _Timer(args.reps)
    d = _setup(args.config)
    rows = _slices_rows(d, timer, (1, 2, 4))
    return {"probe": "recv_slices", "workload": args.config, "n_eff": round(d["n_eff"], 1),
            "active_experts": d["active_experts"], "reps": args.reps, "rows": rows}


# Combine's output store: the library picks sc1 above 256 MiB of combine
# bytes and write-back below; these builds force one form at every size.
COMBINE_STORE_FORMS = {"sc1 at every size": "0", "write-back at every size": "INT64_MAX"}


def _combine_variant(form):
    tag = "sc1" if COMBINE_STORE_FORMS[form] == "0" else "wb"
    return f"combine_store_{tag}", (f"MOE_COMBINE_SC1_MIN_BYTES={COMBINE_STORE_FORMS[form]}",)


def probe_combine_store(args):
    """moe_combine of the library against the builds that force sc1 or
    write-back output stores, on every workload: warm (right after a recv of
    the same workload, as in a step) and cold (after the read sweep)."""
    import torch

    import combine_topk_route_amd as m
    import workloads
    from combine_topk_route_amd import _lib

    fns = {"library (by size)": m._lib.load().moe_combine}
    for form in COMBINE_STORE_FORMS:
        name, defines = _combine_variant(form)
        from combine_topk_route_amd import build as b

        path = b.variant_path(name)
        if not os.path.exists(path):
            b.build_variant(name, defines)
        lib = ctypes.CDLL(path)
        res, argt = _lib.SIGNATURES["moe_combine"]
        lib.moe_combine.restype, lib.moe_combine.argtypes = res, argt
        fns[form] = lib.moe_combine
    timer = _Timer(args.reps)
    out = []
    for name in workloads.CONFIGS:
        d = _setup(name)
        cfg = d["cfg"]
        st = timer.stream.cuda_stream
        s = d["send"]
        ref = m.moe_combine(d["y"], s.pair_row, d["w"])
        recv = lambda: m.moe_dispatch_recv(d["x"], s.pair_row, buf=d["buf"], stream=timer.stream)
        nb = 2 * cfg.P * cfg.H + 8 * cfg.P + 2 * cfg.T * cfg.H
        rows = []
        for label, fn in fns.items():
            call = lambda: fn(d["y"].data_ptr(), s.pair_row.data_ptr(), d["w"].data_ptr(), cfg.T,
                              cfg.H, cfg.k, cfg.P, d["out"].data_ptr(), st)
            d["out"].zero_()
            rc = call()
            torch.cuda.synchronize()
            same = rc == 0 and torch.equal(d["out"].view(torch.int16), ref.view(torch.int16))
            warm = timer.median_us(call, recv)
            cold = timer.median_us(call, timer.cold)
            rows.append({"variant": label, "bit_exact": bool(same), "warm_us": round(warm, 2),
                         "cold_us": round(cold, 2),
                         "warm_frac": round(nb / warm / 1e3 / 8000.0, 4),
                         "cold_frac": round(nb / cold / 1e3 / 8000.0, 4)})
            print(f"[probe] {name} {label}: warm {warm:.2f} us cold {cold:.2f} us",
                  file=sys.stderr, flush=True)
        out.append({"workload": name, "bytes": nb, "rows": rows})
        del d, ref
        torch.cuda.empty_cache()
    return {"probe": "combine_store", "reps": args.reps, "workloads": out}


def probe_store_policy(args):
    timer = _Timer(args.reps)
    d = _setup(args.config)
    variants = [("global nt (library)", None, ())]
    variants += [(form, *_store_variant(form)) for form in STORE_FORMS]
    rows = _variant_rows(d, timer, variants)
    return {"probe": "store_policy", "workload": args.config, "n_eff": round(d["n_eff"], 1),
            "reps": args.reps, "rows": rows}


# Streaming kernels for the practical HBM ceilings (16-byte accesses, 256
# threads per block, grid-stride).  chunk_write / chunk_read: wave w of the
# grid writes / reads chunk order[w] of the buffer (kib KiB, one 16-byte
# access per lane per KiB), so the host sets the pattern: chunks in order,
# or a random permutation.
CEILING_SRC = r"""
#include <hip/hip_runtime.h>
#include <cstdint>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void stream_write(u32x4* __restrict__ d, int64_t n) {
  const u32x4 val = {1u, 2u, 3u, 4u};
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    if (NT) __builtin_nontemporal_store(val, &d[i]); else d[i] = val;
  }
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ s, int64_t n,
                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0u;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const u32x4 v = NT ? __builtin_nontemporal_load(&s[i]) : s[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // keeps the loads; the data never matches
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_copy(const u32x4* __restrict__ s,
                                                   u32x4* __restrict__ d, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const u32x4 v = s[i];
    if (NT) __builtin_nontemporal_store(v, &d[i]); else d[i] = v;
  }
}

__global__ __launch_bounds__(256) void chunk_write(u32x4* __restrict__ d,
                                                   const int32_t* __restrict__ order,
                                                   int64_t nchunks, int kib) {
  const int64_t w = int64_t(blockIdx.x) * 4 + threadIdx.x / 64;
  if (w >= nchunks) return;
  const int64_t c = order[w];
  const u32x4 val = {5u, 6u, 7u, 8u};
  const int lane = threadIdx.x % 64;
  for (int s = 0; s < kib; ++s) __builtin_nontemporal_store(val, &d[(c * kib + s) * 64 + lane]);
}

__global__ __launch_bounds__(256) void chunk_read(const u32x4* __restrict__ s,
                                                  const int32_t* __restrict__ order,
                                                  int64_t nchunks, int kib,
                                                  uint32_t* __restrict__ sink) {
  const int64_t w = int64_t(blockIdx.x) * 4 + threadIdx.x / 64;
  if (w >= nchunks) return;
  const int64_t c = order[w];
  const int lane = threadIdx.x % 64;
  uint32_t acc = 0u;
  for (int q = 0; q < kib; ++q) {
    const u32x4 v = __builtin_nontemporal_load(&s[(c * kib + q) * 64 + lane]);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[w & 1023] = acc;  // keeps the loads; the data never matches
}

extern "C" int ceiling_launch(int op, void* a, void* b, int64_t n16, int64_t blocks,
                              void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g{static_cast<unsigned>(blocks)}, t{256u};
  switch (op) {
    case 0: hipLaunchKernelGGL(stream_write<true>, g, t, 0, st, (u32x4*)a, n16); break;
    case 1: hipLaunchKernelGGL(stream_write<false>, g, t, 0, st, (u32x4*)a, n16); break;
    case 2: hipLaunchKernelGGL(stream_read<true>, g, t, 0, st, (const u32x4*)a, n16, (uint32_t*)b); break;
    case 3: hipLaunchKernelGGL(stream_read<false>, g, t, 0, st, (const u32x4*)a, n16, (uint32_t*)b); break;
    case 4: hipLaunchKernelGGL(stream_copy<true>, g, t, 0, st, (const u32x4*)a, (u32x4*)b, n16); break;
    case 5: hipLaunchKernelGGL(stream_copy<false>, g, t, 0, st, (const u32x4*)a, (u32x4*)b, n16); break;
    case 6: {  // blocks: KiB per chunk
      const int64_t nchunks = n16 / (64 * blocks);
      hipLaunchKernelGGL(chunk_write, dim3(unsigned((nchunks + 3) / 4)), t, 0, st, (u32x4*)a,
                         (const int32_t*)b, nchunks, int(blocks));
      break;
    }
    case 7: {  // chunk reads; b: [order | sink], blocks: KiB per chunk
      const int64_t nchunks = n16 / (64 * blocks);
      hipLaunchKernelGGL(chunk_read, dim3(unsigned((nchunks + 3) / 4)), t, 0, st,
                         (const u32x4*)a, (const int32_t*)b, nchunks, int(blocks),
                         (uint32_t*)b + nchunks);
      break;
    }
    default: return 2;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
"""

CEILING_OPS = {0: "write, nt stores", 1: "write, plain stores", 2: "read, nt loads",
               3: "read, plain loads", 4: "copy, nt stores", 5: "copy, plain stores"}


def _ceiling_lib():
    from combine_topk_route_amd import build as b

    path = b.variant_path("hbm_ceiling", "libhbm_ceiling.so")
    if not os.path.exists(path):
        src = os.path.join(os.path.dirname(path), "hbm_ceiling.hip")
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(src, "w") as f:
            f.write(CEILING_SRC)
        b.build_variant("hbm_ceiling", (), src=src, lib="libhbm_ceiling.so")
    lib = ctypes.CDLL(path)
    lib.ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    lib.ceiling_launch.restype = ctypes.c_int
    return lib


def probe_hbm_ceiling(args):
    """Back-to-back launches over 4 GiB buffers (16 times the Infinity
    Cache): read, write and copy at several grid sizes, and chunk writes and
    reads of 1-16 KiB in order against a random permutation of the chunks."""
    import numpy as np
    import torch

    lib = _ceiling_lib()
    st = torch.cuda.current_stream()
    size = 4 << 30
    n16 = size // 16
    a = torch.empty(size, dtype=torch.uint8, device="cuda")
    b = torch.empty(size, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")

    def timed(op, x, y, blocks):
        for _ in range(3):
            assert lib.ceiling_launch(op, x, y, n16, blocks, st.cuda_stream) == 0
        ev = []
        for _ in range(args.reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            assert lib.ceiling_launch(op, x, y, n16, blocks, st.cuda_stream) == 0
            e1.record(st)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) * 1000.0 for e0, e1 in ev]))

    assert lib.ceiling_launch(0, a.data_ptr(), None, n16, 8192, st.cuda_stream) == 0
    rows = []
    for blocks in (2048, 8192, 32768, 131072):
        for op, name in CEILING_OPS.items():
            y = sink.data_ptr() if op in (2, 3) else b.data_ptr()
            us = timed(op, a.data_ptr(), y, blocks)
            nbytes = size * (2 if op in (4, 5) else 1)
            rows.append({"op": name, "blocks": blocks, "us": round(us, 1),
                         "TBps": round(nbytes / us / 1e6, 3)})
            print(f"[probe] {name} {blocks} blocks: {nbytes / us / 1e6:.2f} TB/s", file=sys.stderr,
                  flush=True)
    rng = np.random.default_rng(0)
    for kib in (1, 2, 4, 8, 14, 16):
        nchunks = size // (1024 * kib)
        used = nchunks * 1024 * kib
        for order_name, order in (("in order", np.arange(nchunks, dtype=np.int32)),
                                  ("random order", rng.permutation(nchunks).astype(np.int32))):
            # the order, then 1024 words of sink for the reads
            o = torch.zeros(nchunks + 1024, dtype=torch.int32, device="cuda")
            o[:nchunks] = torch.from_numpy(order).cuda()
            for op, what in ((6, "writes"), (7, "reads")):
                us = timed(op, a.data_ptr(), o.data_ptr(), kib)
                rows.append({"op": f"{kib} KiB chunk {what}, {order_name}",
                             "blocks": (nchunks + 3) // 4, "us": round(us, 1),
                             "TBps": round(used / us / 1e6, 3)})
                print(f"[probe] {kib} KiB chunk {what} {order_name}: {used / us / 1e6:.2f} TB/s",
                      file=sys.stderr, flush=True)
            del o
    return {"probe": "hbm_ceiling", "bytes": size, "reps": args.reps, "rows": rows}


def probe_skew(args):
    import torch

    timer = _Timer(args.reps)
    out = []
    for s in (None, 0.4, 0.8, 1.2):
        d = _setup("dsv3_prefill", zipf_s=s)
        rows = _slices_rows(d, timer, (1, 2))
        out.append({"zipf_s": s, "n_eff": round(d["n_eff"], 1),
                    "active_experts": d["active_experts"], "rows": rows})
        del d
        torch.cuda.empty_cache()
    return {"probe": "skew", "workload": "dsv3_prefill shape, Zipf routing", "reps": args.reps,
            "sweep": out}


def probe_write_fronts(args):
    import torch

    import combine_topk_route_amd as m

    d = _setup(args.config)
    cfg = d["cfg"]
    adj = torch.arange(cfg.P, dtype=torch.int32, device="cuda").view(cfg.T, cfg.k)
    pr = d["send"].pair_row
    st = torch.cuda.current_stream()
    order = []
    for kern, rows in (("recv", pr), ("recv", adj), ("combine", pr), ("combine", adj)):
        for _ in range(args.launches):
            if kern == "recv":
                m.moe_dispatch_recv(d["x"], rows, buf=d["buf"], stream=st)
            else:
                m.moe_combine(d["y"], rows, d["w"], out=d["out"], stream=st)
            order.append(f"{kern}_{'real' if rows is pr else 'adjacent'}")
        torch.cuda.synchronize()
    return {"probe": "write_fronts", "workload": args.config, "dispatch_order": order}


def _hip_runtime():
    """The HIP runtime torch loaded (the library binds to the same one)."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("libamdhip64 is not loaded")


def probe_cu_scaling(args):
    import torch

    import combine_topk_route_amd as m

    hip = _hip_runtime()
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    d = _setup(args.config)
    cfg = d["cfg"]
    timer = _Timer(args.reps)
    rows = []
    for layout in ("spread", "first"):
        for n in sorted({32, 64, 128, 192, ncu}):
            if n > ncu:
                continue
            cus = ([int(i * ncu / n) for i in range(n)] if layout == "spread" else list(range(n)))
            words = (ctypes.c_uint32 * ((ncu + 31) // 32))()
            for c in cus:
                words[c // 32] |= 1 << (c % 32)
            h = ctypes.c_void_p()
            rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(words), words)
            if rc != 0:
                rows.append({"layout": layout, "cus": n, "error": int(rc)})
                continue
            s = torch.cuda.ExternalStream(h.value)
            timer.stream = s
            with torch.cuda.stream(s):
                call = lambda: m.moe_dispatch_recv(d["x"], d["send"].pair_row, buf=d["buf"],
                                                   stream=s)
                comb = lambda: m.moe_combine(d["y"], d["send"].pair_row, d["w"], out=d["out"],
                                             stream=s)
                warm = timer.median_us(call, comb)
            torch.cuda.synchronize()
            hip.hipStreamDestroy(h)
            nb = _recv_bytes(cfg)
            rows.append({"layout": layout, "cus": n, "warm_us": round(warm, 1),
                         "GBps": round(nb / warm / 1e3, 1),
                         "GBps_per_cu": round(nb / warm / 1e3 / n, 2)})
            print(f"[probe] cu_scaling {layout} {n} CUs: {warm:.1f} us", file=sys.stderr,
                  flush=True)
    return {"probe": "cu_scaling", "workload": args.config, "cus_total": ncu, "reps": args.reps,
            "rows": rows}


def _masked_stream(hip, ncu, first, count):
    """A default-priority stream restricted to CU mask bits [first, first + count)."""
    words = (ctypes.c_uint32 * ((ncu + 31) // 32))()
    for c in range(first, first + count):
        words[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(words), words)
    return (h, rc)


def probe_overlap_masked(args):
    """Dispatch (send + recv) beside the stand-in shared-expert GEMM of
    bench.py's overlap leg, x[T, H] @ W[H, 2048] in bf16: back to back on the
    whole chip, concurrently on two unmasked streams, and concurrently with
    the CUs split between them (dispatch on mask bits [0, n), the GEMM on
    [n, all))."""
    import numpy as np
    import torch

    import combine_topk_route_amd as m

    hip = _hip_runtime()
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    d = _setup(args.config)
    cfg = d["cfg"]
    wsh = torch.randn((cfg.H, 2048), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gout = torch.empty((cfg.T, 2048), dtype=torch.bfloat16, device="cuda")
    main = torch.cuda.current_stream()

    def disp(st):
        m.moe_dispatch(d["idx"], d["x"], cfg.E, cfg.R, buf=d["buf"], stream=st)

    def gemm(st):
        with torch.cuda.stream(st):
            torch.matmul(d["x"], wsh, out=gout)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        res = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(main)
            fn()
            b.record(main)
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) * 1000.0)
        return float(np.median(res))

    def both(s1, s2):
        def fn():
            e = torch.cuda.Event()
            e.record(main)
            s1.wait_event(e)
            s2.wait_event(e)
            disp(s1)
            gemm(s2)
            main.wait_stream(s1)
            main.wait_stream(s2)
        return fn

    reps = args.reps
    t_d = timed(lambda: disp(main), reps)
    t_g = timed(lambda: gemm(main), reps)
    other1, other2 = torch.cuda.Stream(), torch.cuda.Stream()
    t_b = timed(both(other1, other2), reps)
    rows = [{"split": "none (back to back)", "us": round(t_d + t_g, 1)},
            {"split": "two unmasked streams", "us": round(t_b, 1)}]
    for n in (64, 96, 128, 160, 192):
        h1, rc1 = _masked_stream(hip, ncu, 0, n)
        h2, rc2 = _masked_stream(hip, ncu, n, ncu - n)
        if rc1 != 0 or rc2 != 0:
            rows.append({"split": f"{n} / {ncu - n} CUs", "error": [int(rc1), int(rc2)]})
            for h, rc in ((h1, rc1), (h2, rc2)):
                if rc == 0:
                    hip.hipStreamDestroy(h)
            continue
        s1, s2 = torch.cuda.ExternalStream(h1.value), torch.cuda.ExternalStream(h2.value)
        t_d1 = timed(lambda: (s1.wait_stream(main), disp(s1), main.wait_stream(s1)), reps)
        t_g2 = timed(lambda: (s2.wait_stream(main), gemm(s2), main.wait_stream(s2)), reps)
        t_both = timed(both(s1, s2), reps)
        torch.cuda.synchronize()
        hip.hipStreamDestroy(h1)
        hip.hipStreamDestroy(h2)
        rows.append({"split": f"{n} / {ncu - n} CUs", "dispatch_alone_us": round(t_d1, 1),
                     "gemm_alone_us": round(t_g2, 1), "us": round(t_both, 1)})
        print(f"[probe] overlap split {n}/{ncu - n}: {t_both:.1f} us", file=sys.stderr, flush=True)
    return {"probe": "overlap_masked", "workload": args.config, "cus_total": ncu,
            "dispatch_us": round(t_d, 1), "gemm_us": round(t_g, 1),
            "gemm": f"[{cfg.T},{cfg.H}] x [{cfg.H},2048] bf16", "reps": reps, "rows": rows}


PROBES = {"recv_slices": probe_recv_slices, "skew": probe_skew,
          "write_fronts": probe_write_fronts, "cu_scaling": probe_cu_scaling,
          "overlap_masked": probe_overlap_masked, "store_policy": probe_store_policy,
          "hbm_ceiling": probe_hbm_ceiling, "combine_store": probe_combine_store}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("probe", choices=list(PROBES) + ["build"])
    ap.add_argument("--config", default="dsv3_prefill")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--launches", type=int, default=3)
    args = ap.parse_args()
    if args.probe == "build":  # the variant libraries, on a machine with hipcc
        from combine_topk_route_amd import build as b

        for name, defines in [_slice_variant(1), _slice_variant(4)] + [
                _store_variant(f) for f in STORE_FORMS] + [
                _combine_variant(f) for f in COMBINE_STORE_FORMS]:
            print(b.build_variant(name, defines, verbose=True), flush=True)
        _ceiling_lib()
        print(b.variant_path("hbm_ceiling", "libhbm_ceiling.so"), flush=True)
        return 0
    import torch

    torch.cuda.set_device(0)
    print(json.dumps(PROBES[args.probe](args)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
