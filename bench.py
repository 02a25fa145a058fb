#!/usr/bin/env python3
"""Benchmark: halo-attention forward (default) or backward on one MI355X.

One step = one halo_attn_fwd launch over one full batch of the workload (all
of the method's steps run inside that launch); with --pass bwd, one
halo_attn_bwd call (all of its kernels) over one full batch.  Without
--workload the forward line is the headline: the large shape (B=8, 8 heads,
128x128, d=32, block 12, halo 3: 18x18 windows), the largest that fits one
GPU, timed with --steps/--warmup, plus a ``per_config`` block with the same
fields for the other HaloNet-stage shapes (early, mid, strided), measured
first with --per-config-steps launches each.  Inputs are seeded synthetic
tensors already resident in HBM; several independent input/output sets are
rotated so the working set exceeds the 256 MB Infinity Cache and every step
reads HBM.  Prints ONE JSON line (rank 0):

  value      TFLOP/s, F = 4*d*r^2 per (query, head) over the full window
  roofline   dominant kernel vs its binding roof: HBM bandwidth (algorithmic
             bytes per launch: k and v once, q at query pixels, out once) or,
             when the flops take longer at the published peaks, the dense
             matrix peak of the dtype; mean launch time measured with HIP
             events on the launch stream
  achievable_hbm  the same achieved rate over a plain device copy's
             measured rate (context beside the spec peak)
  launch_stats  after the timed region: median, p10 and p90 of single
             launches (events between consecutive launches, sets rotating)
             and the mean over as many launches on one input set ("warm":
             a set that fits the Infinity Cache is read from there)
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload on this host (reported, not a target)

Backward (--pass bwd): one step = one halo_attn_bwd call given the forward's
out and per-query lse (computed once per input set before the timed region,
as a training step keeps them from its forward pass).  F = 10*d*r^2 per
(query, head), the five window contractions q.k (recomputed), dout.v, dl.k,
dl.q, p.dout; algorithmic bytes = e*d*B*heads*(2*(H/s)*(W/s) + 5*H*W): q and
dout once at query pixels, k and v once, dq, dk, dv written once (out and
lse, 1/d of that, not counted).  The roofline entry covers the whole
backward call (its kernels' mean time per call over the timed region).

Layer (--pass layer): one step = one halo_attn_layer_fwd call: to_q / to_kv
of every pixel, the attention, head merge and to_out, on activations kept in
a pixel-major channels-last layout (--layout nhwc or blocked), with C = C_out
= heads*d channels.  F = attention flops + 2*pixels*C*3*inner (to_q, to_kv) +
2*out_pixels*inner*C_out (to_out); algorithmic bytes = x read once and y
written once (the intermediates q, k, v and the attention output are not
counted: a layer that never leaves the chip needs none of them).  The
roofline entry covers the whole call as AUTO runs it (``config.kernel_used``:
"fused" for the one-kernel path, else the attention kernel between the
projections); ``paths_us`` times each path the call can take (split, fused)
and ``parts_us`` each of the split path's three kernels alone.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "halo-attn fwd TFLOP/s + tokens/s per MI355X; % of MFMA/HBM roofline"
METRIC_BWD = "halo-attn bwd TFLOP/s + tokens/s per MI355X; % of MFMA/HBM roofline"
METRIC_LAYER = "halo-attn layer fwd (projections + attention) TFLOP/s + tokens/s per MI355X; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense matrix peaks, published
MALL_BYTES = 256 * 2 ** 20     # Infinity Cache

# HBM bytes per launch of the dominant kernel, per workload: rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the ratio of
# known bytes to the same counter's reading for a plain device copy
# (--copy-calibration).  A record holds only for the kernel it was measured
# on (forward: ``kernel`` = the launched kernel's name) and that kernel's
# sources at the time (``sources`` = kernel_source_hash()); otherwise the
# bench reports traffic as null.
MEASURED_TRAFFIC = {
    "fwd": {
        "large_bf16_128x128_d32_b12h3": {"bytes_per_launch": 273520414, "read": 206411550, "write": 67108864,
            "kernel": "tile", "sources": "75593cc36274afea"},
        "strided_bf16_64x64_d16_b8h3_s2": {"bytes_per_launch": 92520360, "read": 84131752, "write": 8388608,
            "kernel": "ring", "sources": "aa21a7f49d15e703"},
        "early_stage_bf16_64x64_d16_b8h3": {"bytes_per_launch": 134551673, "read": 100997241, "write": 33554432,
            "kernel": "ring", "sources": "aa21a7f49d15e703"},
        "mid_stage_bf16_32x32_d32_b8h3": {"bytes_per_launch": 135622814, "read": 101019806, "write": 34603008,
            "kernel": "ring", "sources": "aa21a7f49d15e703"},
        "detection_bf16_64x64_d16_b32h3": {"bytes_per_launch": 33729341, "read": 25340733, "write": 8388608,
            "kernel": "wide", "sources": "270953bdef674c85"},
        "global_bf16_16x16_d16_b16h0": {"bytes_per_launch": 17115746, "read": 12921442, "write": 4194304,
            "kernel": "ring", "sources": "aa21a7f49d15e703"},
    },
    # layer: summed over the call's kernels (to_q/to_kv, attention, to_out)
    "layer": {
        "early_stage_bf16_64x64_d16_b8h3/nhwc": {"bytes_per_launch": 337275684, "read": 169503524, "write": 167772160,
            "kernel": "ring", "sources": "9b0d378c69acfb61"},
        # the one-kernel path (--layer-kernel fused)
        "early_stage_bf16_64x64_d16_b8h3/nhwc/fused": {"bytes_per_launch": 90591270, "read": 57036838,
            "write": 33554432, "kernel": "fused", "sources": "6889ab74a2b8b934"},
    },
    # backward: summed over the call's kernels (matrix-core kernels, table reduction)
    "bwd": {
        "early_stage_bf16_64x64_d16_b8h3": {"bytes_per_launch": 590464100, "read": 373439460, "write": 217024640,
            "kernel": "strip", "sources": "9c5d4cb0bea600b2"},
        "mid_stage_bf16_32x32_d32_b8h3": {"bytes_per_launch": 504286531, "read": 313506883, "write": 190779648,
            "kernel": "strip", "sources": "9c5d4cb0bea600b2"},
        "strided_bf16_64x64_d16_b8h3_s2": {"bytes_per_launch": 456777508, "read": 260372279, "write": 196405229,
            "kernel": "strip", "sources": "9c5d4cb0bea600b2"},
        "large_bf16_128x128_d32_b12h3": {"bytes_per_launch": 966202901, "read": 689031509, "write": 277171392,
            "kernel": "tile", "sources": "9de16dbfa5ffb275"},
    },
}


# Sources the timed kernels are built from, per pass (the traffic record of
# a pass holds while these files are unchanged).
KERNEL_SOURCES = {
    # forward: per kernel (the record also names the kernel, so a change of
    # kernel selection voids it too)
    "fwd:tile": ["halo_common.h", "mfma_util.h", "kernel_tile.hip"],
    "fwd:ring": ["halo_common.h", "mfma_util.h", "kernel_ring.hip"],
    "fwd:wide": ["halo_common.h", "mfma_util.h", "kernel_wide.hip"],
    "fwd:strip": ["halo_common.h", "mfma_util.h", "kernel_mfma.hip"],
    "fwd:generic": ["halo_common.h", "kernel_generic.hip"],
    # layer: the projections plus the attention kernel the call launches
    "layer:tile": ["halo_common.h", "mfma_util.h", "kernel_tile.hip", "proj.h", "kernel_proj.hip"],
    "layer:ring": ["halo_common.h", "mfma_util.h", "kernel_ring.hip", "proj.h", "kernel_proj.hip"],
    "layer:fused": ["halo_common.h", "mfma_util.h", "proj.h", "kernel_layer.hip"],
    # backward: the matrix-core kernels of the path plus the table reduction
    "bwd:strip": ["halo_common.h", "mfma_util.h", "kernel_bwd_mfma.hip", "kernel_bwd_generic.hip"],
    "bwd:tile": ["halo_common.h", "mfma_util.h", "kernel_bwd_tile.hip", "kernel_bwd_generic.hip"],
    "bwd:generic": ["halo_common.h", "kernel_generic.hip", "kernel_bwd_generic.hip"],
}


def kernel_source_hash(which: str = "fwd") -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[which]:
        h.update(name.encode())
        with open(os.path.join(HERE, "blocked_local_self_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--issue-rates", action="store_true",
                    help="time the library's issue-rate probe (FMA, exp2, MFMA, mixed waves) instead")
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed launches first (the GPU clocks need ~0.1 s of load to ramp up)")
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the forward headline is the large 18x18-window shape, "
                         "reported with every HaloNet-stage shape; the backward and layer passes default "
                         "to the early-stage shape)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "mfma", "mfma_ring", "mfma_strip"])
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd", "layer"],
                    help="forward (the headline), backward pass, or the whole layer with its projections")
    ap.add_argument("--layout", default="nhwc", choices=["nhwc", "blocked"],
                    help="activation layout of --pass layer")
    ap.add_argument("--layer-kernel", default="auto", choices=["auto", "fused", "split"],
                    help="path of --pass layer's timed calls (halo_attn_layer_fwd_ex kernel)")
    ap.add_argument("--variants", default="", help="comma-separated semantic variants of the forward "
                    "(centred_offset, zero_pad, centred_mask, half_split); default: none")
    ap.add_argument("--sets", type=int, default=0, help="rotated input sets (0: enough to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle sample time")
    ap.add_argument("--per-config-steps", type=int, default=500,
                    help="timed launches per stage shape in the per_config block (after as many warm-up launches)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run --steps plain device copies of MIB MiB each "
                         "(the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    import torch
    n = mib * 2 ** 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n, "bytes_written_per_copy": n,
                                           "copies": steps}}), flush=True)


def issue_rates(iters=8000):
    """Per-SIMD issue rates of the instruction kinds the attention kernels
    are made of, from the library's probe kernel (halo_attn_probe_issue):
    each mode's launch is timed with HIP events (10 launches after 3), the
    rate is wave-instructions per SIMD per second, also given as SIMD cycles
    per wave-instruction at the 2.4 GHz spec clock.  The mixed modes put two
    instruction kinds in the two halves of every workgroup (waves sharing a
    SIMD): their time is compared with the sum and the maximum of the two
    halves' times alone."""
    import torch
    from blocked_local_self_amd import _native
    lib = _native.load()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    simds = 4 * cus
    wgs = 4 * cus
    waves = 8 * wgs
    out = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch_ms(mode):
        for _ in range(3):
            _native.check(lib.halo_attn_probe_issue(mode, iters, wgs, out.data_ptr(), stream.cuda_stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(10):
            lib.halo_attn_probe_issue(mode, iters, wgs, out.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 10

    t = {m: launch_ms(m) for m in range(6)}
    per_wave = {0: 8 * iters, 1: 8 * iters, 2: 4 * iters, 3: 4 * iters}
    kinds = {0: "fma_f32", 1: "exp2_f32", 2: "mfma_16x16x32_bf16", 3: "mfma_32x32x16_bf16"}
    res = {"simds": simds, "waves": waves, "iters": iters}
    for m, name in kinds.items():
        per_simd = waves * per_wave[m] / simds
        rate = per_simd / (t[m] * 1e-3)
        res[name] = {"launch_ms": round(t[m], 4), "wave_instr_per_simd_per_s": round(rate, 1),
                     "cycles_per_wave_instr_at_2.4GHz": round(2.4e9 / rate, 2)}
    res["mfma_16x16x32_bf16"]["tflops"] = round(waves * per_wave[2] * 16384 / (t[2] * 1e-3) / 1e12, 1)
    res["mfma_32x32x16_bf16"]["tflops"] = round(waves * per_wave[3] * 32768 / (t[3] * 1e-3) / 1e12, 1)
    res["exp_over_fma_time"] = round(t[1] / t[0], 3)
    for m, (a, b, name) in {4: (1, 2, "exp_with_mfma_16x16x32"), 5: (1, 0, "exp_with_fma")}.items():
        res[name] = {"launch_ms": round(t[m], 4), "sum_of_halves_ms": round((t[a] + t[b]) / 2, 4),
                     "max_of_halves_ms": round(max(t[a], t[b]) / 2, 4)}
    print(json.dumps({"issue_rates": res}), flush=True)


def device_info():
    """The GPU the line was measured on (name, architecture, compute units)."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "cus": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2 ** 30, 1)}


def copy_bandwidth_gbs(mib=512, reps=10):
    """Achievable HBM bandwidth as context for the spec peak: a plain device
    copy (torch copy_) of `mib` MiB, event-timed over `reps` copies after two
    untimed ones; bytes = read + written."""
    import torch
    n = mib * 2 ** 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def with_copy_context(e, copy_gbs):
    """Add the achieved HBM rate as a fraction of the measured copy rate."""
    r = e.get("roofline", {})
    if r.get("bound") == "hbm":
        e["achievable_hbm"] = {"copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(r["achieved"] / copy_gbs, 4),
                               "what": "torch copy_ of 512 MiB on the same GPU, read + written bytes"}
    return e


def bwd_flops(wl):
    return 10 * wl.d * wl.r * wl.r * wl.B * wl.heads * wl.Ho * wl.Wo


def bwd_alg_bytes(wl):
    return wl.elem_bytes * wl.d * wl.B * wl.heads * (2 * wl.Ho * wl.Wo + 5 * wl.H * wl.W)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inputs_cpu, target_s, dout_cpu=None):
    """Time the fp64 oracle on whole (batch, head) slices of the workload.

    The sample grows (more slices, then repeated passes over all of them)
    until it holds about ``target_s`` seconds of CPU work.
    """
    import numpy as np
    import oracle
    f64 = lambda t: t.to(dtype=__import__("torch").float64).numpy()
    q, k, v, rh, rw = (f64(t) for t in inputs_cpu)
    g = f64(dout_cpu) if dout_cpu is not None else None
    threads = oracle.max_threads()
    nslices = wl.B * wl.heads
    per_slice_flops = (wl.flops if g is None else bwd_flops(wl)) / nslices

    def run(nsl):
        sl = lambda a: np.ascontiguousarray(a.reshape(nslices, 1, *a.shape[2:])[:nsl])
        args = [sl(q), sl(k), sl(v)]
        t0 = time.perf_counter()
        if g is None:
            oracle.halo_attn_ref(*args, rh, rw, wl.block, wl.halo, wl.stride, threads=threads)
        else:
            oracle.halo_attn_bwd_ref(*args, rh, rw, sl(g), wl.block, wl.halo, wl.stride, threads=threads)
        return time.perf_counter() - t0

    n = min(threads, nslices)
    t = run(n)
    if t < target_s and n < nslices:
        n2 = int(min(nslices, n * target_s / max(t, 1e-3)))
        n2 = max(n, (n2 // threads) * threads) if n2 >= threads else n2
        if n2 > n:
            n, t = n2, run(n2)
    passes = 1
    while t < target_s and n == nslices and passes < 200:
        t += run(n)
        passes += 1
    flops = per_slice_flops * n * passes
    tokens = wl.tokens * n * passes / nslices   # token = output position with all heads
    what = f"{n} of {nslices} (batch, head) slices" if n < nslices else f"all {nslices} (batch, head) slices"
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of {wl.name} x {passes} pass(es), {'backward' if g is not None else 'forward'}, "
                      f"fp64, {t:.2f} s",
            "seconds": round(t, 3), "tokens_per_s": round(tokens / t, 1), "cpu_model": cpu_model()}


def layer_flops(wl, C, Co):
    inner = wl.heads * wl.d
    return wl.flops + 2 * wl.B * wl.H * wl.W * C * 3 * inner + 2 * wl.B * wl.Ho * wl.Wo * inner * Co


def layer_alg_bytes(wl, C, Co):
    return wl.elem_bytes * (wl.B * wl.H * wl.W * C + wl.B * wl.Ho * wl.Wo * Co)


def cpu_baseline_layer(wl, xs, target_s):
    """Time the fp64 oracle layer on whole images of the workload."""
    import oracle
    f64 = lambda t: t.to(dtype=__import__("torch").float64).numpy()
    x, w_q, w_kv, w_o, b_o, rh, rw = (f64(t) for t in xs)
    C = x.shape[-1]
    Co = w_o.shape[0]
    threads = oracle.max_threads()
    per_image = layer_flops(wl, C, Co) / wl.B
    n, t, images = 1, 0.0, 0
    while t < target_s and images < 64 * wl.B:
        sl = x[(images % wl.B):(images % wl.B) + n]
        t0 = time.perf_counter()
        oracle.halo_layer_ref(sl, w_q, w_kv, w_o, b_o, rh, rw, wl.block, wl.halo, wl.heads, wl.stride,
                              threads=threads)
        t += time.perf_counter() - t0
        images += sl.shape[0]
        n = min(wl.B, 2 * n)
    return {"value": round(per_image * images / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{images} images of {wl.name} (layer: projections + attention, C={C}), fp64, {t:.2f} s",
            "seconds": round(t, 3), "tokens_per_s": round(wl.tokens / wl.B * images / t, 1)}


def run_layer(args):
    import torch
    from blocked_local_self_amd import (halo_layer_fwd, halo_layer_proj_in, halo_layer_proj_out, halo_attn_fwd,
                                        layer_workspace_bytes, workloads, _native, LAYOUTS)
    from blocked_local_self_amd.inputs import make_layer_inputs, nhwc_to_layout

    wl = workloads.get(args.workload or workloads.PASS_WORKLOAD)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    C = Co = wl.heads * wl.d
    inner = wl.heads * wl.d
    lay = args.layout
    side, side_o = wl.block, wl.block // wl.stride
    e = wl.elem_bytes
    per_set = e * (wl.B * wl.H * wl.W * C + wl.B * wl.Ho * wl.Wo * Co)
    nsets = args.sets or max(2, -(-2 * MALL_BYTES // per_set))
    sets = []
    xs0 = None
    for s_ in range(nsets):
        xs = make_layer_inputs(wl.B, wl.H, wl.W, C, wl.heads, wl.d, wl.block, wl.halo, dtype=wl.dtype, seed=s_)
        if s_ == 0:
            xs0 = xs
        dt = [nhwc_to_layout(xs[0], lay, side).to(dev)] + [t.to(dev) for t in xs[1:]]
        ys = (wl.B, wl.Ho, wl.Wo, Co) if lay == "nhwc" else (wl.B, wl.Ho // side_o, wl.Wo // side_o, side_o ** 2, Co)
        sets.append((dt, torch.empty(ys, dtype=dt[0].dtype, device=dev)))
    nws = layer_workspace_bytes(wl.B, wl.H, wl.W, wl.heads, wl.d, wl.stride, wl.dtype)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = _native.load()
    dcode = _native.HALO_BF16 if wl.dtype == "bf16" else _native.HALO_F32
    scale = float(wl.d) ** -0.5
    calls = []
    for (x, w_q, w_kv, w_o, b_o, rh, rw), y in sets:
        halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, wl.block, wl.halo, wl.heads, wl.stride, layout=lay,
                       workspace=ws, out=y, stream=stream)
        calls.append((x.data_ptr(), w_q.data_ptr(), w_kv.data_ptr(), w_o.data_ptr(), b_o.data_ptr(), rh.data_ptr(),
                      rw.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), wl.B, wl.H, wl.W, C, Co, wl.heads,
                      wl.d, wl.block, wl.halo, wl.stride, scale, LAYOUTS[lay], dcode, stream.cuda_stream))

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0

    lk = {"auto": _native.HALO_LAYER_KERNEL_AUTO, "fused": _native.HALO_LAYER_KERNEL_FUSED,
          "split": _native.HALO_LAYER_KERNEL_SPLIT}[args.layer_kernel]

    def step(i):
        st = lib.halo_attn_layer_fwd_ex(*calls[i % nsets][:-1], lk, calls[i % nsets][-1])
        if st:
            _native.check(st)

    ms, wall = timed(step, args.steps, args.warmup)

    # each path of the call on its own (AUTO above takes one of them)
    dcode_ = _native.HALO_BF16 if wl.dtype == "bf16" else _native.HALO_F32
    paths = {}
    for pname, pcode in (("split", _native.HALO_LAYER_KERNEL_SPLIT), ("fused", _native.HALO_LAYER_KERNEL_FUSED)):
        try:
            _native.layer_kernel_name(wl.B, wl.H, wl.W, C, Co, wl.heads, wl.d, wl.block, wl.halo, wl.stride,
                                      LAYOUTS[lay], dcode_, kernel=pcode)
        except ValueError:
            continue

        def step_path(i, pcode=pcode):
            st = lib.halo_attn_layer_fwd_ex(*calls[i % nsets][:-1], pcode, calls[i % nsets][-1])
            if st:
                _native.check(st)

        paths[pname] = timed(step_path, max(10, args.steps // 4), 20)[0]
    # the three kernels of the split path on their own (same shapes and layout)
    (x, w_q, w_kv, w_o, b_o, rh, rw), y = sets[0]
    q, k, v = halo_layer_proj_in(x, w_q, w_kv, wl.heads, side, lay, stream=stream)
    attn = halo_attn_fwd(q, k, v, rh, rw, wl.block, wl.halo, wl.stride, stream=stream)
    parts = {}
    nsteps = max(10, args.steps // 4)
    parts["proj_in"] = timed(lambda i: halo_layer_proj_in(sets[i % nsets][0][0], w_q, w_kv, wl.heads, side, lay,
                                                          stream=stream), nsteps, 20)[0]
    parts["attention"] = timed(lambda i: halo_attn_fwd(q, k, v, rh, rw, wl.block, wl.halo, wl.stride, out=attn,
                                                       stream=stream), nsteps, 20)[0]
    parts["proj_out"] = timed(lambda i: halo_layer_proj_out(attn, w_o, b_o, side_o, lay, stream=stream),
                              nsteps, 20)[0]

    flops = layer_flops(wl, C, Co)
    alg_bytes = layer_alg_bytes(wl, C, Co)
    tflops = flops / (ms * 1e-3) / 1e12
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    mfma_peak = MFMA_PEAK_TFLOPS[wl.dtype]
    mfma_bound = flops / (mfma_peak * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9)
    used = _native.layer_kernel_name(wl.B, wl.H, wl.W, C, Co, wl.heads, wl.d, wl.block, wl.halo, wl.stride,
                                     LAYOUTS[lay], dcode_, kernel=lk)
    if used == "split":     # named by the attention kernel between the projections
        used = _native.fwd_kernel_name(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride, dcode_)
    src_hash = kernel_source_hash(f"layer:{used}") if f"layer:{used}" in KERNEL_SOURCES else None
    rec = MEASURED_TRAFFIC["layer"].get(f"{wl.name}/{lay}" + ("/fused" if used == "fused" else ""))
    valid = rec is not None and src_hash is not None and rec["sources"] == src_hash and rec.get("kernel") == used
    traffic = rec["bytes_per_launch"] if valid else None
    line = {
        "metric": METRIC_LAYER, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {**wl.describe(), "pass": "layer", "kernel_used": used, "layout": lay, "C": C, "C_out": Co,
                   "rotated_input_sets": nsets},
        "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(tflops, 2) if mfma_bound else round(achieved_gbs, 1),
            "peak": mfma_peak if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(tflops / mfma_peak if mfma_bound else achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes,
            "flops_per_launch": flops,
            "mean_launch_us": round(ms * 1e3, 3),
            "kernel_sources": src_hash,
        },
        "paths_us": {k_: round(v_ * 1e3, 3) for k_, v_ in paths.items()},
        "parts_us": {k_: round(v_ * 1e3, 2) for k_, v_ in parts.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_layer(wl, xs0, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the operation shards over batch x heads with no communication)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.issue_rates:
        issue_rates()
        return
    if args.which == "layer":
        run_layer(args)
        return
    import torch
    from blocked_local_self_amd import workloads
    if args.which == "bwd" or args.workload or args.variants:
        wl = workloads.get(args.workload or (workloads.PASS_WORKLOAD if args.which == "bwd"
                                             else workloads.BENCH_WORKLOAD))
        print(json.dumps(run_op(args, wl, args.steps, args.warmup, args.cpu_seconds)), flush=True)
        return
    # the forward headline: the inputs of every HaloNet-stage shape are put
    # on the GPU first; then each stage shape is timed (with its own
    # warm-up) and the headline shape last with the requested steps, back to
    # back; the CPU baselines follow once the GPU work is done
    names = [n for n in workloads.STAGE_WORKLOADS if n != workloads.BENCH_WORKLOAD]
    prepared = {n: prepare_op(args, workloads.get(n)) for n in names + [workloads.BENCH_WORKLOAD]}
    per_config = {}
    for name in names:
        e = prepared[name][0](args.per_config_steps, args.per_config_steps)
        per_config[name] = {k_: e[k_] for k_ in ("value", "unit", "ms_per_step", "tokens_per_s", "dtype", "steps",
                                                  "warmup", "roofline", "launch_stats", "config")}
    line = prepared[workloads.BENCH_WORKLOAD][0](args.steps, args.warmup)
    if not args.no_cpu_baseline:
        for name in names:
            per_config[name]["cpu_baseline"] = prepared[name][1](min(5.0, args.cpu_seconds))
        line["cpu_baseline"] = prepared[workloads.BENCH_WORKLOAD][1](args.cpu_seconds)
    prepared.clear()
    torch.cuda.empty_cache()
    copy_gbs = copy_bandwidth_gbs()
    with_copy_context(line, copy_gbs)
    for e in per_config.values():
        with_copy_context(e, copy_gbs)
    line["per_config"] = per_config
    print(json.dumps(line), flush=True)


def run_op(args, wl, steps, warmup, cpu_seconds):
    """Time `steps` launches of the forward (or backward) on workload wl after
    `warmup` untimed ones; returns the JSON line's fields."""
    measure, cpu_job = prepare_op(args, wl)
    line = measure(steps, warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_job(cpu_seconds)
    return line


def prepare_op(args, wl):
    """Inputs of workload wl resident on the GPU and the launch arguments;
    returns (measure(steps, warmup) -> the JSON line's fields without the
    CPU baseline, cpu_job(seconds) -> the CPU baseline), so that several
    workloads can be prepared first and timed back to back (the GPU then
    stays busy, and its clocks up, from one timed region to the next)."""
    import torch
    from blocked_local_self_amd import halo_attn_fwd, halo_attn_bwd, bwd_workspace_bytes, workloads
    from blocked_local_self_amd.inputs import make_workload_inputs, make_grad_output

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    in_bytes = 3 * wl.elem_bytes * wl.B * wl.heads * wl.H * wl.W * wl.d
    out_bytes = wl.elem_bytes * wl.B * wl.heads * wl.Ho * wl.Wo * wl.d
    bwd = args.which == "bwd"
    variants = tuple(v for v in args.variants.split(",") if v)
    if variants and bwd:
        print("--variants applies to the forward pass only", file=sys.stderr)
        sys.exit(2)
    per_set = in_bytes + out_bytes if not bwd else 2 * in_bytes + 2 * out_bytes
    nsets = args.sets or max(2, -(-2 * MALL_BYTES // per_set))
    sets = []
    inputs0_cpu = dout0_cpu = None
    for s in range(nsets):
        cpu = make_workload_inputs(wl, seed=s)
        if s == 0:
            inputs0_cpu = cpu
        dev_t = tuple(t.to(dev) for t in cpu)
        if bwd:
            g_cpu = make_grad_output(wl.B, wl.heads, wl.Ho, wl.Wo, wl.d, dtype=wl.dtype, seed=s)
            if s == 0:
                dout0_cpu = g_cpu
            q, k, v, rh, rw = dev_t
            fwd = halo_attn_fwd(q, k, v, rh, rw, wl.block, wl.halo, wl.stride, kernel=args.kernel,
                                return_lse=True)
            sets.append((dev_t, (g_cpu.to(dev),) + fwd))
        else:
            sets.append((dev_t, torch.empty(wl.out_shape(), dtype=dev_t[0].dtype, device=dev)))
    stream = torch.cuda.current_stream(dev)
    ws = None
    if bwd:
        nws = bwd_workspace_bytes(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride, wl.dtype)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        grads = tuple(torch.empty(wl.shape(), dtype=sets[0][0][0].dtype, device=dev) for _ in range(3)) + \
            tuple(torch.empty((2 * wl.r - 1, wl.d), dtype=torch.float32, device=dev) for _ in range(2))

    # Every input set goes once through the checked torch-level wrapper; the
    # timed steps then call the same C entry point with the argument tuples
    # prepared here, so host-side argument checking does not pace the GPU
    # (it would for the smallest workloads).
    from blocked_local_self_amd import _native, KERNELS, VARIANTS
    lib = _native.load()
    dcode = _native.HALO_BF16 if wl.dtype == "bf16" else _native.HALO_F32
    flags = sum(VARIANTS[v] for v in variants)
    scale = float(wl.d) ** -0.5
    calls = []
    for (q, k, v, rh, rw), x in sets:
        if bwd:
            g, out, lse = x
            halo_attn_bwd(q, k, v, rh, rw, g, wl.block, wl.halo, wl.stride, out=out, lse=lse,
                          kernel=args.kernel, workspace=ws, grads=grads, stream=stream)
            calls.append((lib.halo_attn_bwd_kernel,
                          (q.data_ptr(), k.data_ptr(), v.data_ptr(), rh.data_ptr(), rw.data_ptr(), out.data_ptr(),
                           g.data_ptr(), lse.data_ptr(), *[t.data_ptr() for t in grads], ws.data_ptr(),
                           ws.numel(), wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride, scale,
                           dcode, KERNELS[args.kernel], stream.cuda_stream)))
        else:
            halo_attn_fwd(q, k, v, rh, rw, wl.block, wl.halo, wl.stride, out=x, kernel=args.kernel,
                          stream=stream, variants=variants)
            calls.append((lib.halo_attn_fwd_ex,
                          (q.data_ptr(), k.data_ptr(), v.data_ptr(), rh.data_ptr(), rw.data_ptr(), x.data_ptr(),
                           None, wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride, scale, dcode,
                           flags, KERNELS[args.kernel], stream.cuda_stream)))

    def step(i):
        fn, a = calls[i % nsets]
        st = fn(*a)
        if st:
            _native.check(st)

    def measure(steps, warmup):
        return _measure(args, wl, step, stream, nsets, lib, dcode, flags, variants, bwd, steps, warmup)

    def cpu_job(seconds):
        return cpu_baseline(wl, inputs0_cpu, seconds, dout0_cpu)

    return measure, cpu_job


def _measure(args, wl, step, stream, nsets, lib, dcode, flags, variants, bwd, steps, warmup):
    import torch
    from blocked_local_self_amd import _native, KERNELS
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms = gpu_ms / steps

    # Spread of single launches (outside the timed region above): a chain of
    # events between consecutive launches on the same stream, the input sets
    # rotating as above; then `steps` launches on input set 0 alone ("warm":
    # when a set fits the 256 MB Infinity Cache, its reads hit there).
    nsamp = max(1, min(steps, 200))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsamp + 1)]
    evs[0].record(stream)
    for i in range(nsamp):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(nsamp))
    pick = lambda f: per_launch[min(nsamp - 1, int(f * (nsamp - 1) + 0.5))]
    ev0.record(stream)
    for i in range(steps):
        step(0)
    ev1.record(stream)
    torch.cuda.synchronize()
    launch_stats = {"median_us": round(pick(0.5), 3), "p10_us": round(pick(0.1), 3),
                    "p90_us": round(pick(0.9), 3), "samples": nsamp,
                    "warm_mean_us": round(ev0.elapsed_time(ev1) * 1e3 / steps, 3)}
    flops = bwd_flops(wl) if bwd else wl.flops
    alg_bytes = bwd_alg_bytes(wl) if bwd else wl.alg_bytes
    tflops = flops / (ms * 1e-3) / 1e12
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    # the binding roof: whichever of HBM bytes and matrix flops takes longer
    # at the published peaks
    mfma_peak = MFMA_PEAK_TFLOPS[wl.dtype]
    mfma_bound = flops / (mfma_peak * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9)

    if bwd:
        used = _native.bwd_kernel_name(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride, dcode,
                                       flags, KERNELS[args.kernel])
        src_hash = kernel_source_hash(f"bwd:{used}")
    else:
        used = _native.fwd_kernel_name(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride, dcode,
                                       flags, KERNELS[args.kernel])
        src_hash = kernel_source_hash(f"fwd:{used}")
    rec = None if variants else MEASURED_TRAFFIC[args.which].get(wl.name)
    valid = rec is not None and rec["sources"] == src_hash and rec.get("kernel") == used
    traffic = rec["bytes_per_launch"] if valid else None

    line = {
        "metric": METRIC_BWD if bwd else METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {**wl.describe(), "pass": args.which, "kernel": args.kernel,
                   **({"kernel_used": used} if used else {}), "rotated_input_sets": nsets,
                   **({"variants": list(variants)} if variants else {})},
        "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(tflops, 2) if mfma_bound else round(achieved_gbs, 1),
            "peak": mfma_peak if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(tflops / mfma_peak if mfma_bound else achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes,
            "mean_launch_us": round(ms * 1e3, 3),
            "kernel_sources": src_hash,
        },
        "launch_stats": launch_stats,
        "device": device_info(),
    }
    return line




if __name__ == "__main__":
    main()
