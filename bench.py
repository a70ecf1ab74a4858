#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE decode layer on one MI355X.

Metric: microseconds per MoE layer and achieved HBM GB/s (fraction of the
8 TB/s peak).  A step is one moe_decode_layer call -- router, top-k, shared
expert, routed experts FC1/FC2 and the combine -- on one batch of synthetic
rows of the K3-shaped layer (hidden 7168, 896 experts, top-16, intermediate
1536, 17,547,264-byte MXFP4 experts, bf16 shared expert), batch 1.

Cache hygiene: MI355X has 256 MB of last-level cache (MALL) and a step reads
~360 MB, so consecutive steps rotate over `--layers` distinct copies of the
layer (each 15.7 GB of experts) and over `--variants` input rows (different
routing), so no step finds its weights in cache from an earlier step.
Bytes are algorithmic: router + shared expert + U distinct experts (counted
from each step's actual routing) + activations.

Prints ONE JSON line.  `value` is algorithmic bytes over the wall time of K
steps launched back to back.  `roofline` is for the dominant kernel -- the
layer is a single persistent kernel, k_moe_layer -- whose average launch
duration is the span of two HIP events recorded on the launch stream around
those K launches, divided by K.  Every timed step is then re-run alone and
must reproduce its residual bit for bit (`validated`).  `cpu_baseline` is the
CPU oracle on one batch-1 layer, on all host threads and on one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

PEAK_GBPS = 8000.0
METRIC = "µs per MoE layer and achieved HBM GB/s (% of peak) at batch 1/8/64"


def layer_bytes(cfg, idx, with_bias: bool):
    """Algorithmic HBM bytes of one layer step, total and per kernel."""
    import numpy as np
    import synth
    H, I, E, k, Is = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.shared_inter
    B = idx.shape[0]
    U = int(np.unique(idx).size)
    nb = synth.expert_bytes(H, I)
    router = E * H * 2 + (E * 4 if with_bias else 0)
    shared = 3 * Is * H * 2
    act = B * (H * 2 + 2 * H * 4)  # x read, residual read + write
    total = router + shared + U * nb + act
    # the layer is one kernel: its algorithmic bytes are the layer's
    per_kernel = {"k_moe_layer": total}
    return {"total": total, "U": U, "per_kernel": per_kernel}


def _step_args(lib, w, x, res, idx, gate, ws, stream):
    """The ctypes argument tuple of one moe_decode_layer call (built outside the
    timed loop, so the loop costs one foreign call per step)."""
    import ctypes
    import memory_bound_mxfp4_amd as moe
    cs = w.c_struct()
    return (ctypes.byref(cs), moe._ptr(x), moe._ptr(res), x.shape[0], moe._ptr(idx), moe._ptr(gate), moe._ptr(ws),
            ws.numel(), moe._stream(stream)), cs


def _pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v, np.float64), q))


CLOCK_WARMUP_S = 0.3


def run_config(cfg, layers, steps, warmup, variants, seed=0, event_reps=None, mxfp8=False,
               clock_warmup_s=CLOCK_WARMUP_S):
    """Times `steps` layer steps launched back to back, then checks them.

    * clock warm-up: `clock_warmup_s` seconds of untimed steps, then the W
      warm-up steps;
    * timed pass: K steps enqueued back to back (one foreign call each);
      wall clock between two synchronisations, and two HIP events recorded on
      the launch stream before the first and after the last launch (the GPU
      span, which the host's launch rate cannot stretch once the queue is
      ahead of the GPU);
    * validation: the workspace status word must read 0, and every timed
      step's residual and indices must be bit-identical to the same step
      re-run alone (synchronised) on the same inputs -- a launch that
      overlapped its predecessor or took stale data would differ;
    * per-launch events: `event_reps` more launches, each bracketed by events
      recorded by the library, for the median / p10 / p90 of one launch.
    mxfp8: time moe_decode_layer_mxfp8 (FP4 x MXFP8 routed experts) instead.
    """
    import numpy as np
    import torch

    import memory_bound_mxfp4_amd as moe
    from layer_inputs import residual_from_x, x_host
    lib = moe.load()
    B = cfg.batch
    names = moe.layer_kernel_names()
    xs = [torch.from_numpy(x_host(cfg, seed, variant=v)).cuda() for v in range(variants)]
    res0 = [torch.from_numpy(residual_from_x(x_host(cfg, seed, variant=v))).cuda() for v in range(variants)]
    total = warmup + steps
    res = [res0[s % variants].clone() for s in range(total)]
    idx = torch.empty((total, B, cfg.top_k), dtype=torch.int32, device="cuda")
    gate = torch.empty((total, B, cfg.top_k), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(layers[0], B)
    bias = None
    if cfg.zipf_s is not None:
        import synth
        bias = torch.from_numpy(synth.zipf_bias(seed, 0, cfg.num_experts, cfg.zipf_s)).cuda()
    saved_bias = [w.router_bias for w in layers]
    for w in layers:
        w.router_bias = bias
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    event_reps = steps if event_reps is None else event_reps
    try:
        args, keep = [], []
        for s in range(total):
            a, cs = _step_args(lib, layers[s % len(layers)], xs[s % variants], res[s], idx[s], gate[s], ws, stream)
            args.append(a)
            keep.append(cs)
        call = lib.moe_decode_layer_mxfp8 if mxfp8 else lib.moe_decode_layer
        # Clock warm-up: after an idle spell the first ~100 launches run while
        # the GPU clocks ramp up from their idle state (7-8% slower); untimed
        # steps for `clock_warmup_s` bring them to their steady state first.
        r_w = res0[0].clone()  # the warm-up steps' own residual (the timed steps' inputs stay untouched)
        wargs = []
        for j in range(len(layers)):
            a, cs = _step_args(lib, layers[j], xs[j % variants], r_w, idx[0], gate[0], ws, stream)
            wargs.append(a)
            keep.append(cs)
        t_w = time.perf_counter()
        n_w = 0
        while time.perf_counter() - t_w < clock_warmup_s:
            assert call(*wargs[n_w % len(wargs)]) == moe.MOE_OK
            n_w += 1
            if n_w % 64 == 0:
                torch.cuda.synchronize()
        for s in range(warmup):
            assert call(*args[s]) == moe.MOE_OK
        torch.cuda.synchronize()
        # Timed pass: K steps launched back to back (the throughput `value`).
        t0 = time.perf_counter()
        e0.record(stream)
        for s in range(warmup, total):
            call(*args[s])
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        status = moe.workspace_status(ws)
        # Validation: each timed step again, alone, from the same inputs.
        mismatches = 0
        for i in range(steps):
            s = warmup + i
            r_v = res0[s % variants].clone()
            i_v = torch.empty_like(idx[s])
            g_v = torch.empty_like(gate[s])
            moe.moe_decode_layer(layers[s % len(layers)], xs[s % variants], r_v, idx=i_v, gate=g_v, ws=ws,
                                 mxfp8=mxfp8)
            torch.cuda.synchronize()
            same = torch.equal(r_v.view(torch.int32), res[s].view(torch.int32)) and torch.equal(i_v, idx[s])
            mismatches += 0 if same else 1
        status = status | moe.workspace_status(ws)
        # Per-launch events (the library records them around its kernel).
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(event_reps)]
        for i in range(event_reps):
            s = warmup + i % steps
            r_e = res0[s % variants].clone()
            if mxfp8:  # one kernel: events recorded around the call on the launch stream
                ev[i][0].record(stream)
                moe.moe_decode_layer(layers[s % len(layers)], xs[s % variants], r_e, idx=idx[s], gate=gate[s], ws=ws,
                                     stream=stream, mxfp8=True)
                ev[i][1].record(stream)
            else:
                moe.moe_decode_layer_timed(layers[s % len(layers)], xs[s % variants], r_e, idx[s], gate[s], ws,
                                           ev[i], stream=stream)
        torch.cuda.synchronize()
    finally:
        for w, b in zip(layers, saved_bias):
            w.router_bias = b
    wall_s = t1 - t0
    span_ms = e0.elapsed_time(e1)
    idx_h = idx[warmup:].cpu().numpy()
    per = [layer_bytes(cfg, idx_h[i], bias is not None) for i in range(steps)]
    tot_bytes = sum(p["total"] for p in per)
    launch_us = {n: [ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(event_reps)]
                 for j, n in enumerate(names)}
    kb = {n: float(np.mean([p["per_kernel"][n] for p in per])) for n in per[0]["per_kernel"]}
    return {
        "wall_s": wall_s,
        "us_per_layer": wall_s / steps * 1e6,
        "gpu_span_us_per_layer": span_ms / steps * 1e3,
        "gbps": tot_bytes / wall_s / 1e9,
        "gbps_gpu_span": tot_bytes / (span_ms * 1e-3) / 1e9,
        "bytes_per_layer": tot_bytes / steps,
        "U_mean": float(np.mean([p["U"] for p in per])),
        "U_min": int(min(p["U"] for p in per)),
        "U_max": int(max(p["U"] for p in per)),
        "kernel_bytes": kb,
        "launch_us": {n: {"median": round(_pct(v, 50), 2), "p10": round(_pct(v, 10), 2), "p90": round(_pct(v, 90), 2),
                          "reps": len(v)} for n, v in launch_us.items()},
        "validated": {"status_word": int(status), "steps_bit_identical_to_serial_rerun": steps - mismatches,
                      "steps": steps, "ok": status == 0 and mismatches == 0},
    }


KERNEL_SOURCES = ("layer.hip", "moe_device.h", "mx_common.h", "internal.h", "api.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_moe_layer_k3_b1_traffic.txt")
CALIB_BYTES = 256 << 20  # plain device-to-device copy used to scale the HBM byte counters


def kernel_source_hash() -> str:
    """sha256 over the sources the layer kernel is compiled from and the
    compiler flags it is built with."""
    import hashlib
    from memory_bound_mxfp4_amd import build as _build
    h = hashlib.sha256()
    h.update(" ".join(_build.FLAGS).encode())
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "memory_bound_mxfp4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def calibration_copy():
    """One copy of CALIB_BYTES (read CALIB_BYTES, write CALIB_BYTES), outside any
    timed region: a kernel of known traffic that counter runs scale by."""
    import torch
    a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def recorded_traffic():
    """HBM bytes per k_moe_layer launch measured by counters (profiles file), or
    None when the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return int(rec["traffic_bytes_per_launch"])


def pmc_summary(fetch_csv, write_csv, kernel="k_moe_layer"):
    """Scaled HBM traffic of `kernel` from FETCH_SIZE and WRITE_SIZE counter CSVs
    (rocprofv3 --pmc ... --output-format csv).  Each counter is scaled by the
    ratio of the calibration copy's known bytes to what the counter read for it."""
    import csv
    import numpy as np

    def per_kernel(path, counter):
        vals, calib = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            if kernel in name:
                vals.append(v)
            elif "copyBuffer" in name:
                calib.append(v)  # the runtime's copy kernel; the largest dispatch is the calibration copy
        return vals, calib
    f_vals, f_cal = per_kernel(fetch_csv, "FETCH_SIZE")
    w_vals, w_cal = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = CALIB_BYTES / (max(f_cal) * 1024)
    w_scale = CALIB_BYTES / (max(w_cal) * 1024)
    fetch = float(np.mean(f_vals)) * 1024 * f_scale
    write = float(np.mean(w_vals)) * 1024 * w_scale
    return {"fetch_kib_raw": float(np.mean(f_vals)), "write_kib_raw": float(np.mean(w_vals)),
            "calib_fetch_kib": max(f_cal), "calib_write_kib": max(w_cal), "fetch_scale": f_scale,
            "write_scale": w_scale, "fetch_bytes": int(fetch), "write_bytes": int(write),
            "traffic_bytes_per_launch": int(fetch + write), "dispatches": len(f_vals),
            "kernel_source_hash": kernel_source_hash()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seed=0):
    """The oracle on one K3-shaped batch-1 layer, once on one thread and once
    on every host thread (its expert evaluations spread by OpenMP); expert
    regeneration excluded.  About 7 s of CPU time on this class of host."""
    import oracle
    from layer_inputs import host_experts, host_weights, residual_from_x, x_host
    from synth import CONFIGS
    cfg = CONFIGS["k3_b1"]
    hw = host_weights(cfg, seed)
    x = x_host(cfg, seed)
    res = residual_from_x(x)
    lg, _ = oracle.router_logits(x, hw["router_w"], None, cfg.hidden, cfg.num_experts)
    idx, _ = oracle.topk(lg, cfg.top_k)
    experts = host_experts(cfg, seed, idx.ravel())
    nproc = os.cpu_count() or 1
    n_all = oracle.set_threads(0)
    times = {}
    try:
        for n in (1, n_all):
            oracle.set_threads(n)
            t0 = time.perf_counter()
            r = oracle.moe_layer(cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.shared_inter, hw["router_w"],
                                 None, hw["shared_gate"], hw["shared_up"], hw["shared_down"], experts, x, res)
            times[n] = time.perf_counter() - t0
    finally:
        oracle.set_threads(n_all)
    nbytes = layer_bytes(cfg, r["idx"], False)["total"]
    return {"value": round(nbytes / times[n_all] / 1e9, 4), "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "us_per_layer": round(times[n_all] * 1e6, 1),
            "single_thread": {"value": round(nbytes / times[1] / 1e9, 4), "us_per_layer": round(times[1] * 1e6, 1)},
            "host": {"nproc": nproc, "cpu_model": _cpu_model(), "omp_threads": n_all},
            "sample": "one K3-shaped batch-1 layer (hidden 7168, 896 experts, top-16, seed 0): router + top-k + "
                      "shared + 16 routed experts + combine; value on `cores` threads (17 independent expert "
                      "evaluations spread by OpenMP), single_thread on one; expert regeneration excluded"}


def stream_ceiling(gib=4, reps=8):
    """The device's streaming-read rate (moe_stream_read_probe over `gib` GiB,
    best of a few grid shapes, median over `reps` reads each): context for the
    layer's fraction of the 8 TB/s peak."""
    import numpy as np
    import torch

    import memory_bound_mxfp4_amd as moe
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = (0.0, 0)
    for bpc in (2, 4, 8):
        moe.stream_read_probe(buf, bpc, sink)
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            moe.stream_read_probe(buf, bpc, sink)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        gbps = nbytes / (float(np.median(ts)) * 1e-3) / 1e9
        if gbps > best[0]:
            best = (gbps, bpc)
    del buf
    return {"gbps": round(best[0], 1), "frac_of_peak": round(best[0] / PEAK_GBPS, 4), "bytes": nbytes,
            "blocks_per_cu": best[1], "kernel": "k_stream_read (moe_stream_read_probe)"}


def dense_gemv_times(batches=(1, 8, 64), mats=8, reps=24):
    """dense_gemv_bf16 on 7168 x 7168 bf16 matrices (the stack's dense block),
    rotating over `mats` distinct matrices so none is read from cache; median
    per-launch event time per batch."""
    import numpy as np
    import torch

    import memory_bound_mxfp4_amd as moe
    import synth
    from synth import CONFIGS
    cfg = CONFIGS["k3_stack8"]
    H = cfg.hidden
    Ws = []
    for j in range(mats):
        t = torch.empty((H, H), dtype=torch.int16, device="cuda")
        synth.dev_fill_bf16(t, 0, synth.tag(0, synth.KIND_DENSE, 0, j), cfg.weight_sigma)
        Ws.append(t.view(torch.bfloat16))
    out = {}
    for B in batches:
        x = torch.randn((B, H), device="cuda").to(torch.bfloat16)
        y = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
        for W in Ws[:2]:
            moe.dense_gemv_bf16(W, x, y=y)
        ts = []
        for i in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            moe.dense_gemv_bf16(Ws[i % mats], x, y=y)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        us = float(np.median(ts))
        nbytes = H * H * 2 + B * H * 2 * 2
        out[f"b{B}"] = {"us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    del Ws
    return out


def run_stack(stack, steps, warmup, graph=True, seed=0):
    """Times decode steps of the 8-layer stack (dense block + MoE layer per
    layer), captured in one HIP graph per step when `graph`."""
    import numpy as np
    import torch

    import synth
    from layer_inputs import h0_host
    cfg = stack_cfg()
    h0 = torch.from_numpy(h0_host(cfg, seed)).cuda()
    h = h0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(1, warmup)):
            stack.step(h, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            stack.step(h, stream=s)
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    idx = []
    with torch.cuda.stream(s):
        t_w = time.perf_counter()  # clock warm-up (untimed), as for the single layer
        while time.perf_counter() - t_w < CLOCK_WARMUP_S:
            if g is not None:
                g.replay()
            else:
                stack.step(h, stream=s)
            s.synchronize()
        e0.record(s)
        for _ in range(steps):
            if g is not None:
                g.replay()
            else:
                stack.step(h, stream=s)
        e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    idx_h = stack.idx.cpu().numpy()  # routing of the last step
    H = cfg.hidden
    nb = synth.expert_bytes(H, cfg.inter)
    per_layer = [cfg.num_experts * H * 2 + 3 * cfg.shared_inter * H * 2 + int(np.unique(idx_h[l]).size) * nb +
                 cfg.batch * (H * 2 + 2 * H * 4) + cfg.dense_mats * (H * H * 2 + cfg.batch * 4 * H) +
                 2 * cfg.batch * (H * 4 + H * 2 + H * 4)
                 for l in range(cfg.layers)]
    step_bytes = sum(per_layer)
    return {"us_per_step": ms * 1e3, "us_per_layer": ms * 1e3 / cfg.layers, "bytes_per_step": step_bytes,
            "gbps": step_bytes / (ms * 1e-3) / 1e9, "graph": g is not None,
            "kernels_per_step": cfg.layers * (cfg.dense_mats + 4)}


def stack_cfg():
    from synth import CONFIGS
    return CONFIGS["k3_stack8"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer copies rotated across steps")
    ap.add_argument("--variants", type=int, default=32, help="distinct input rows rotated across steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other batch sizes")
    ap.add_argument("--extra", default="k3_b4,k3_b8,k3_b16,k3_b64_zipf,k3_b8_mxfp8,k3_b64_zipf_mxfp8",
                    help="comma-separated other batch configurations to time (_mxfp8: moe_decode_layer_mxfp8)")
    ap.add_argument("--no-stack", action="store_true", help="skip the 8-layer decode-step stack line")
    ap.add_argument("--no-probe", action="store_true", help="skip the stream-read ceiling and dense GEMV lines")
    ap.add_argument("--stack-prefetch", default="none",
                    help="comma-separated side-stream prefetch modes of the stack to time (none, dense, moe, both)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the scaled HBM traffic of k_moe_layer from two counter CSVs and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        for k, v in pmc_summary(*args.pmc_summary).items():
            print(f"{k} = {v}")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the layer fits one MI355X; "
              "there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    from dataclasses import replace
    from layer_inputs import dense_device, device_weights
    from synth import CONFIGS
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = CONFIGS["k3_b1"]
    n_layers = max(args.layers, 0 if args.no_stack else stack_cfg().layers)
    print(f"[bench] generating {n_layers} K3-shaped layers in HBM", file=sys.stderr, flush=True)
    layers = [device_weights(cfg, 0, layer=l) for l in range(n_layers)]
    calibration_copy()
    print("[bench] timing batch 1", file=sys.stderr, flush=True)
    main_r = run_config(cfg, layers[:args.layers], args.steps, args.warmup, args.variants)
    extra = {}
    if not args.no_extra:
        b8 = CONFIGS["k3_b8"]
        wanted = set(args.extra.split(","))
        for name, c in (("k3_b4", replace(b8, name="k3_b4", batch=4)), ("k3_b8", b8),
                        ("k3_b16", replace(b8, name="k3_b16", batch=16)), ("k3_b64_zipf", CONFIGS["k3_b64_zipf"]),
                        ("k3_b8_mxfp8", b8), ("k3_b64_zipf_mxfp8", CONFIGS["k3_b64_zipf"])):
            if name not in wanted:
                continue
            print(f"[bench] timing {name}", file=sys.stderr, flush=True)
            r = run_config(c, layers[:args.layers], max(20, args.steps // 2), args.warmup, args.variants,
                           mxfp8=name.endswith("_mxfp8"))
            extra[name] = {"batch": c.batch, "us_per_layer": round(r["us_per_layer"], 2),
                           "gbps": round(r["gbps"], 1), "frac_peak": round(r["gbps"] / PEAK_GBPS, 4),
                           "gpu_span_us_per_layer": round(r["gpu_span_us_per_layer"], 2),
                           "distinct_experts": round(r["U_mean"], 1), "launch_us_events": r["launch_us"],
                           "validated": r["validated"]}
    if not args.no_stack:
        from memory_bound_mxfp4_amd.stack import DecodeStack
        sc = stack_cfg()
        print("[bench] timing the 8-layer decode-step stack", file=sys.stderr, flush=True)
        dense = [dense_device(sc, 0, l) for l in range(sc.layers)]
        for mode in args.stack_prefetch.split(","):
            stack = DecodeStack(layers[:sc.layers], dense, sc.batch, sc.rms_eps, prefetch=mode)
            r = run_stack(stack, max(5, args.steps // 6), 2)
            key = "k3_stack8" if mode == "none" else f"k3_stack8_prefetch_{mode}"
            extra[key] = {"batch": sc.batch, "layers": sc.layers, "us_per_step": round(r["us_per_step"], 1),
                          "us_per_layer": round(r["us_per_layer"], 2), "gbps": round(r["gbps"], 1),
                          "frac_peak": round(r["gbps"] / PEAK_GBPS, 4), "bytes_per_step": r["bytes_per_step"],
                          "hip_graph": r["graph"], "kernels_per_step": r["kernels_per_step"], "prefetch": mode}
            del stack
        del dense
    probe = dense = None
    if not args.no_probe:
        del layers
        torch.cuda.empty_cache()
        print("[bench] stream-read ceiling and dense GEMV", file=sys.stderr, flush=True)
        probe = stream_ceiling()
        dense = dense_gemv_times()
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    kbytes = main_r["kernel_bytes"]["k_moe_layer"]
    k_us = main_r["gpu_span_us_per_layer"]
    achieved = kbytes / (k_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(main_r["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["us_per_layer"] / 1e3, 5),
        "us_per_layer": round(main_r["us_per_layer"], 2),
        "frac_peak": round(main_r["gbps"] / PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generator; weights ~N(0,0.02), MXFP4 experts, activations ~N(0,1))",
        "config": {"workload": "K3-shaped MoE decode layer, batch 1: hidden 7168, 896 experts, top-16, "
                               "expert intermediate 1536 (MXFP4, 17,547,264 B/expert), bf16 shared expert 1536, "
                               "bf16 router", "batch": 1, "distinct_layers_rotated": args.layers,
                   "input_variants": args.variants, "bytes_per_layer": int(main_r["bytes_per_layer"]),
                   "distinct_experts": round(main_r["U_mean"], 1)},
        "kernels_per_layer": len(main_r["launch_us"]),
        "validated": main_r["validated"],
        "gpu_span_us_per_layer": round(k_us, 2),
        "clock_warmup_s": CLOCK_WARMUP_S,
        "launch_us_events": main_r["launch_us"],
        "roofline": {"kernel": "k_moe_layer", "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "traffic": recorded_traffic(),
                     "algorithmic_bytes_per_launch": int(kbytes), "avg_launch_us": round(k_us, 2),
                     "avg_launch_us_from": "HIP events on the launch stream around the K back-to-back launches, / K",
                     "stream_read_ceiling": probe},
        "cpu_baseline": cpu,
        "extra_configs": extra,
        "dense_gemv_7168x7168": dense,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
