#!/usr/bin/env python3
"""Benchmark of the grouped / depthwise conv forward HIP library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--op fwd]

A step is one pass of the hot path over one batch of every workload in the
set: by default all eight workloads (small fp32 grouped; MobileNetV2-style
depthwise fp16 at stride 1 and 2; ResNeXt-style bf16; 3D grouped fp16 at N=1
and N=8; large-group bf16 with dilation 1 and 2), i.e. eight gconv_fwd calls
per step, each one kernel launch.  Inputs are seeded synthetic tensors
already resident in HBM.  To keep the 256 MB Infinity Cache from serving
repeated reads, every call takes the next of R rotating input / output
buffer sets of its workload, R chosen so the sets span >= 512 MB.

Prints ONE JSON line: whole-step algorithmic HBM throughput (GB/s) as
`value`; per workload, the kernel's average duration from a pair of HIP
events that the library binds to its dispatch (on the launch stream, every
S-th timed step), TFLOP/s, GB/s, both fractions of the MI355X peaks and a
roofline object; `roofline` for the dominant (longest) kernel; and a
`cpu_baseline` object (the CPU oracle, timed on this host's cores on the
first images of every workload).  `traffic` is the HBM bytes per launch from
committed rocprofv3 counters (profiles/traffic.json), null once the kernel's
sources have changed since they were taken.

--op bwd_data / bwd_weight time the backward calls on one workload's shapes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from depthwise_convolution_grouped_amd import inputs, metrics  # noqa: E402

# name -> the workloads whose forward calls make up one step
WORKLOAD_SETS = {"all": list(inputs.WORKLOADS),
                 "depthwise2d_pair": ["depthwise2d_f16", "depthwise2d_s2_f16"]}
for _n in inputs.WORKLOADS:
    WORKLOAD_SETS.setdefault(_n, [_n])

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
ROTATE_BYTES = 512 << 20
LAUNCH_BOUND_BYTES = 8 << 20     # below this a problem's launch costs more than its HBM time


def stored_traffic(workload: str, path_name: str):
    """HBM bytes per launch from committed rocprofv3 counters, if taken on these sources."""
    from depthwise_convolution_grouped_amd.profile_summary import source_hash
    try:
        with open(PROFILE_TRAFFIC) as f:
            db = json.load(f)
    except (OSError, ValueError):
        return None
    e = db.get(workload)
    if not e or e.get("kernel") != path_name or e.get("source_hash") != source_hash(path_name):
        return None
    return e.get("hbm_bytes_per_launch")


class hip_runtime:
    """The HIP runtime the process already uses (the one torch loaded), for
    events that the library binds to a kernel dispatch."""

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.L = ctypes.CDLL(path)
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def event(self) -> int:
        e = self.ct.c_void_p()
        rc = self.L.hipEventCreate(self.ct.byref(e))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed (%d)" % rc)
        self.made.append(e.value)
        return e.value

    def elapsed_ms(self, e0: int, e1: int) -> float:
        ms = self.ct.c_float()
        rc = self.L.hipEventElapsedTime(self.ct.byref(ms), e0, e1)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def destroy_all(self):
        for e in self.made:
            self.L.hipEventDestroy(e)
        self.made = []


def cpu_baseline(names, max_seconds: float):
    """Time the CPU oracle on the first images of every workload of the step,
    each given an equal share of `max_seconds`, on this host's cores."""
    import oracle
    total_bytes, elapsed = 0, 0.0
    per, parts = {}, []
    share = max_seconds / len(names)
    for n in names:
        wl = inputs.WORKLOADS[n]
        p = wl.problem
        t = inputs.workload_tensors(wl)
        x = inputs.storage_to_f64(t.x, p.dtype)
        w = inputs.storage_to_f64(t.w, p.dtype)
        b = inputs.storage_to_f64(t.bias, p.dtype) if t.bias is not None else None
        st, pd, dl = p.spatial_args()
        done, secs, nb = 0, 0.0, 0
        while done == 0 or secs < share:
            # one image first, then as many as the remaining share allows,
            # going round the batch again when it is done
            i0 = done % p.N
            k = 1 if done == 0 else max(1, min(p.N - i0, int((share - secs) / (secs / done))))
            t0 = time.perf_counter()
            oracle.conv_fwd(x[i0:i0 + k], w, b, p.G, st, pd, dl)
            secs += time.perf_counter() - t0
            nb += metrics.total_bytes(_with_batch(p, k))
            done += k
        per[n] = {"gbs": nb / secs / 1e9, "images": done, "seconds": secs}
        parts.append("%s %d images (batch %d)" % (n, done, p.N))
        total_bytes += nb
        elapsed += secs
    return {
        "value": total_bytes / elapsed / 1e9,
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "fp64 direct conv (the oracle), an equal time share per workload, images taken in "
                  "batch order: %s; %.1f s in all"
                  % (", ".join(parts), elapsed),
        "per_config": per,
    }


def _with_batch(p, n):
    return inputs.Problem(p.ndim, p.dtype, n, p.G, p.C, p.K, p.spatial, p.filt, p.stride, p.pad,
                          p.dil, p.bias)


def bwd_problem(p):
    """The workload's problem without bias (backward data has none)."""
    return inputs.Problem(p.ndim, p.dtype, p.N, p.G, p.C, p.K, p.spatial, p.filt, p.stride, p.pad,
                          p.dil, False)


def cpu_baseline_bwd(name, op: str, max_seconds: float):
    """The oracle's backward data or backward weight on this host's cores, on
    the first images of the workload (as many as fit in `max_seconds`)."""
    import oracle
    p = bwd_problem(inputs.WORKLOADS[name].problem)
    t = inputs.make_tensors(p, 4100)
    x = inputs.storage_to_f64(t.x, p.dtype)
    w = inputs.storage_to_f64(t.w, p.dtype)
    o = metrics.out_spatial(p)
    dshape = (p.N,) + (o if p.ndim == 3 else o[1:]) + (p.K,)
    dy = inputs.storage_to_f64(inputs.make_array(dshape, p.dtype, 4105), p.dtype)
    st, pd, dl = p.spatial_args()
    in_sp = p.x_shape()[1:-1]

    def run(k):
        if op == "bwd_data":
            oracle.conv_bwd_data(dy[:k], w, p.G, in_sp, st, pd, dl)
        else:
            oracle.conv_bwd_weight(x[:k], dy[:k], p.G, p.w_shape()[1:-1], st, pd, dl)

    done, secs, nb = 0, 0.0, 0
    while done < p.N and (done == 0 or secs < max_seconds):
        k = 1 if done == 0 else max(1, min(p.N - done, int((max_seconds - secs) / (secs / done))))
        t0 = time.perf_counter()
        run(k)
        secs += time.perf_counter() - t0
        nb += metrics.total_bytes(_with_batch(p, k))
        done += k
    what = "backward data" if op == "bwd_data" else "backward weight"
    return {"value": nb / secs / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%s %s (the oracle, fp64) on the first %d of %d images, %.1f s"
                      % (name, what, done, p.N, secs)}


def bench_bwd_data(a, G, torch):
    """Backward data (gconv_bwd_data) on the first workload of the set: the same
    rotating-buffer protocol, timed with events on the launch stream around
    each call (the stride-1 route is two kernels: weight transform + forward)."""
    name = WORKLOAD_SETS[a.workload][0]
    p = bwd_problem(inputs.WORKLOADS[name].problem)
    dev = torch.device("cuda", 0)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[p.dtype]
    d = G.desc_from_problem(p)
    o = G.gconv_out_dims(d)
    dshape = (p.N,) + (o if p.ndim == 3 else o[1:]) + (p.K,)
    per_set = metrics.io_bytes(p)["x"] + metrics.io_bytes(p)["y"]
    R = 1 if a.hot else min(64, max(2, -(-ROTATE_BYTES // per_set)))
    dy0 = torch.randn(dshape, device=dev, generator=torch.Generator(device=dev).manual_seed(7)).to(tdt)
    dys = [dy0] + [dy0.clone() for _ in range(R - 1)]
    dxs = [torch.empty(p.x_shape(), dtype=tdt, device=dev) for _ in range(R)]
    w = (torch.randn(p.w_shape(), device=dev, generator=torch.Generator(device=dev).manual_seed(8))
         / (p.Cpg * p.filt[0] * p.filt[1] * p.filt[2]) ** 0.5).to(tdt)
    need = G.gconv_bwd_data_workspace(d)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def call(i):
        rc = G.gconv_bwd_data(d, dys[i % R].data_ptr(), w.data_ptr(), dxs[i % R].data_ptr(),
                              ws.data_ptr(), need, sptr)
        if rc != 0:
            raise G.GconvError(rc, "gconv_bwd_data(%s)" % name)

    for i in range(a.warmup):
        call(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for k in range(a.steps):
        evs[k][0].record(stream)
        call(k)
        evs[k][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / a.steps
    ds = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    avg_ms = sum(ds) / len(ds)
    r = metrics.rates(p, avg_ms * 1e-3)
    ai = metrics.flops(p) / metrics.total_bytes(p)
    peak_tf = metrics.PEAK_TFLOPS["f32_vector"] if p.dtype == "f32" else metrics.PEAK_TFLOPS[p.dtype]
    if ai < peak_tf * 1e12 / (metrics.PEAK_HBM_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": r["gbs"], "peak": metrics.PEAK_HBM_GBS, "unit": "GB/s",
                "frac": r["frac_hbm"]}
    else:
        roof = {"bound": "alu" if p.dtype == "f32" else "mfma", "achieved": r["tflops"], "peak": peak_tf,
                "unit": "TFLOP/s", "frac": r["frac_compute"]}
    route = ("weight transform + forward %s" % G.gconv_path_name(G.gconv_select_path(
        G.make_desc(p.ndim, p.dtype, p.N, p.G, p.K, p.C, o if p.ndim == 3 else o[1:],
                    p.filt if p.ndim == 3 else p.filt[1:], (1,) * p.ndim,
                    tuple(p.dil[i] * (p.filt[i] - 1) - p.pad[i] for i in range(3 - p.ndim, 3)),
                    p.spatial_args()[2])))) if need else "direct"
    roof.update({"traffic": stored_traffic("bwd_data:" + name, "bwd_data"),
                 "kernel": "bwd_data (%s)" % route, "workload": name,
                 "algorithmic_bytes": metrics.total_bytes(p), "algorithmic_flop": metrics.flops(p),
                 "us_per_launch": avg_ms * 1e3, "timed_launches": len(ds),
                 "timing": "event pair around each gconv_bwd_data call on the launch stream"})
    out = {
        "metric": "grouped conv bwd_data TFLOP/s + HBM GB/s (% of MI355X peak), 1 GPU",
        "value": metrics.total_bytes(p) / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p.dtype,
        "data": "synthetic (seeded; dy~N(0,1), w~N(0,1/fan_in)); inputs resident in HBM",
        "config": {"workload": inputs.WORKLOADS[name].about + " (backward data, no bias)", "names": [name],
                   "layout": "dy NHWGK, w GKYXC -> dx NHWGC",
                   "cache": "hot (no rotation)" if a.hot else "rotating buffer sets >= 512 MB"},
        "per_config": {name: {"route": route, "us_avg": avg_ms * 1e3, "us_median": ds[len(ds) // 2] * 1e3,
                              "us_min": ds[0] * 1e3, "tflops": r["tflops"], "gbs": r["gbs"],
                              "frac_hbm": r["frac_hbm"], "frac_compute": r["frac_compute"],
                              "rotating_sets": R}},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_bwd(name, "bwd_data", a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def bench_bwd_weight(a, G, torch):
    """Backward weight (gconv_bwd_weight, full partial-sum workspace) on the first
    workload of the set, timed like backward data (events around each call:
    the two-stage reduction is two kernels)."""
    name = WORKLOAD_SETS[a.workload][0]
    p = bwd_problem(inputs.WORKLOADS[name].problem)
    dev = torch.device("cuda", 0)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[p.dtype]
    d = G.desc_from_problem(p)
    o = G.gconv_out_dims(d)
    dshape = (p.N,) + (o if p.ndim == 3 else o[1:]) + (p.K,)
    per_set = metrics.io_bytes(p)["x"] + metrics.io_bytes(p)["y"]
    R = 1 if a.hot else min(64, max(2, -(-ROTATE_BYTES // per_set)))
    gen = torch.Generator(device=dev)
    x0 = torch.randn(p.x_shape(), device=dev, generator=gen.manual_seed(5)).to(tdt)
    dy0 = torch.randn(dshape, device=dev, generator=gen.manual_seed(6)).to(tdt)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    dys = [dy0] + [dy0.clone() for _ in range(R - 1)]
    dw = torch.empty(p.w_shape(), dtype=tdt, device=dev)
    need = G.gconv_bwd_weight_workspace(d)
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def call(i):
        rc = G.gconv_bwd_weight(d, xs[i % R].data_ptr(), dys[i % R].data_ptr(), dw.data_ptr(),
                                ws.data_ptr(), need, sptr)
        if rc != 0:
            raise G.GconvError(rc, "gconv_bwd_weight(%s)" % name)

    for i in range(a.warmup):
        call(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for k in range(a.steps):
        evs[k][0].record(stream)
        call(k)
        evs[k][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / a.steps
    ds = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    avg_ms = sum(ds) / len(ds)
    r = metrics.rates(p, avg_ms * 1e-3)
    # stage 1 runs on the matrix cores for half types (the implicit GEMM over
    # output pixels) and on the vector ALUs for fp32; stage 2 is a short fp32 sum
    peak_tf = metrics.PEAK_TFLOPS["f32_vector"] if p.dtype == "f32" else metrics.PEAK_TFLOPS[p.dtype]
    ai = metrics.flops(p) / metrics.total_bytes(p)
    if ai < peak_tf * 1e12 / (metrics.PEAK_HBM_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": r["gbs"], "peak": metrics.PEAK_HBM_GBS, "unit": "GB/s",
                "frac": r["frac_hbm"]}
    else:
        roof = {"bound": "alu" if p.dtype == "f32" else "mfma", "achieved": r["tflops"], "peak": peak_tf,
                "unit": "TFLOP/s", "frac": r["tflops"] / peak_tf}
    route = "two-stage reduction (%d B of partial sums)" % need if need else "one-stage reduction"
    roof.update({"traffic": stored_traffic("bwd_weight:" + name, "bwd_weight"),
                 "kernel": "bwd_weight (%s)" % route, "workload": name,
                 "algorithmic_bytes": metrics.total_bytes(p), "algorithmic_flop": metrics.flops(p),
                 "us_per_launch": avg_ms * 1e3, "timed_launches": len(ds),
                 "timing": "event pair around each gconv_bwd_weight call on the launch stream"})
    out = {
        "metric": "grouped conv bwd_weight TFLOP/s + HBM GB/s (% of MI355X peak), 1 GPU",
        "value": metrics.total_bytes(p) / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p.dtype,
        "data": "synthetic (seeded; x, dy ~ N(0,1)); inputs resident in HBM",
        "config": {"workload": inputs.WORKLOADS[name].about + " (backward weight)", "names": [name],
                   "layout": "x NHWGC, dy NHWGK -> dw GKYXC",
                   "cache": "hot (no rotation)" if a.hot else "rotating buffer sets >= 512 MB"},
        "per_config": {name: {"route": route, "us_avg": avg_ms * 1e3, "us_median": ds[len(ds) // 2] * 1e3,
                              "us_min": ds[0] * 1e3, "tflops": r["tflops"], "gbs": r["gbs"],
                              "frac_hbm": r["frac_hbm"], "frac_mfma_peak": r["tflops"] / peak_tf,
                              "rotating_sets": R}},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_bwd(name, "bwd_weight", a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def fwd_rooflines(p, us_avg, path_name, key):
    """The roofline object of one forward config: HBM-bound below the ridge
    point of its compute unit, else bound by that unit; launch-bound when the
    whole problem moves less than 8 MB (the launch itself then dominates)."""
    r = metrics.rates(p, us_avg * 1e-6)
    ai = metrics.flops(p) / metrics.total_bytes(p)
    # fp32 runs on the vector ALUs (256 FLOP/clk/CU x 256 CUs x 2.4 GHz =
    # 157.3 TFLOP/s); half types on the matrix cores
    peak_tf = metrics.PEAK_TFLOPS["f32_vector"] if p.dtype == "f32" else metrics.PEAK_TFLOPS[p.dtype]
    ridge = peak_tf * 1e12 / (metrics.PEAK_HBM_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": r["gbs"], "peak": metrics.PEAK_HBM_GBS, "unit": "GB/s",
                "frac": r["gbs"] / metrics.PEAK_HBM_GBS}
    else:
        roof = {"bound": "alu" if p.dtype == "f32" else "mfma", "achieved": r["tflops"],
                "peak": peak_tf, "unit": "TFLOP/s", "frac": r["tflops"] / peak_tf}
    roof["traffic"] = stored_traffic(key, path_name)
    roof["launch_bound"] = metrics.total_bytes(p) < LAUNCH_BOUND_BYTES
    return roof


def bench_fwd(a, G, torch):
    names = WORKLOAD_SETS[a.workload]
    path = G.GCONV_PATH_AUTO if a.path == "auto" else G.PATHS[a.path]
    dev = torch.device("cuda", 0)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

    def to_dev(arr, dtype):
        import numpy as np
        if dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(arr))
        return t.to(dev)

    calls = []
    for n in names:
        wl = inputs.WORKLOADS[n]
        p = wl.problem
        t = inputs.workload_tensors(wl)
        d = G.desc_from_problem(p)
        o = G.gconv_out_dims(d)
        oshape = (p.N,) + (o if p.ndim == 3 else o[1:]) + (p.K,)
        per_set = metrics.io_bytes(p)["x"] + metrics.io_bytes(p)["y"]
        # enough sets to span 512 MB (twice the 256 MB Infinity Cache), at most
        # 64: a workload that small is launch-bound and gains nothing from more
        R = 1 if a.hot else min(64, max(2, -(-ROTATE_BYTES // per_set)))
        x0 = to_dev(t.x, p.dtype)
        xs = [x0] + [x0.clone() for _ in range(R - 1)]
        ys = [torch.empty(oshape, dtype=tdt[p.dtype], device=dev) for _ in range(R)]
        w = to_dev(t.w, p.dtype)
        b = to_dev(t.bias, p.dtype) if t.bias is not None else None
        sel = G.gconv_select_path(d) if path == G.GCONV_PATH_AUTO else path
        calls.append(dict(name=n, p=p, d=d, xs=xs, ys=ys, w=w, b=b, R=R, path=sel,
                          plan=G.gconv_get_plan(d, sel)))

    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    counter = [0]
    hip = hip_runtime()

    def launch(c, e0=None, e1=None):
        # e0/e1: a start/stop event pair (created beforehand) bound to this one dispatch
        i = counter[0] % c["R"]
        rc = G.gconv_fwd_timed(c["d"], c["path"], c["xs"][i].data_ptr(), c["w"].data_ptr(),
                               c["b"].data_ptr() if c["b"] is not None else None,
                               c["ys"][i].data_ptr(), sptr, e0, e1)
        if rc != 0:
            raise G.GconvError(rc, "gconv_fwd(%s)" % c["name"])

    def step(events=None, k=0):
        for c in calls:
            if events is not None:
                launch(c, *events[c["name"]][k])
            else:
                launch(c)
        counter[0] += 1

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps back to back.  The dispatches of every S-th step
    # carry a bound event pair (created before the region); the others are
    # plain launches, so the host stays ahead of the GPU and the step time is
    # the GPU's.
    every = max(1, a.event_every)
    sampled = list(range(0, a.steps, every))
    events = {c["name"]: [(hip.event(), hip.event()) for _ in sampled] for c in calls}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(a.steps):
        if k % every == 0:
            step(events, k // every)
        else:
            step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / a.steps

    per_config = {}
    step_bytes = 0
    step_flops = 0
    for c in calls:
        ds = sorted(hip.elapsed_ms(e0, e1) for e0, e1 in events[c["name"]])
        avg_ms = sum(ds) / len(ds)
        p = c["p"]
        r = metrics.rates(p, avg_ms * 1e-3)
        name = G.gconv_path_name(c["path"])
        roof = fwd_rooflines(p, avg_ms * 1e3, name, c["name"])
        per_config[c["name"]] = {
            "path": name,
            "us_avg": avg_ms * 1e3, "us_median": ds[len(ds) // 2] * 1e3, "us_min": ds[0] * 1e3,
            "tflops": r["tflops"], "gbs": r["gbs"], "frac_hbm": r["frac_hbm"],
            "frac_compute": r["frac_compute"], "flop": metrics.flops(p),
            "bytes": metrics.total_bytes(p), "rotating_sets": c["R"],
            "grid": list(c["plan"]["grid"]), "block": c["plan"]["block"],
            "roofline": roof,
        }
        step_bytes += metrics.total_bytes(p)
        step_flops += metrics.flops(p)
    hip.destroy_all()

    # the dominant kernel: the config with the longest kernel time per step
    dominant = max(per_config, key=lambda n: per_config[n]["us_avg"])
    dom = per_config[dominant]
    dp = inputs.WORKLOADS[dominant].problem
    roof = dict(dom["roofline"])
    roof.update({"kernel": dom["path"], "workload": dominant,
                 "algorithmic_bytes": metrics.total_bytes(dp), "algorithmic_flop": metrics.flops(dp),
                 "us_per_launch": dom["us_avg"], "timed_launches": len(sampled),
                 "timing": "event pair bound to the dispatch (hipExtLaunchKernel) on every %d-th timed "
                           "step, on the launch stream" % every})
    dtypes = sorted({inputs.WORKLOADS[n].problem.dtype for n in names})
    out = {
        "metric": "grouped conv fwd TFLOP/s + HBM GB/s (% of MI355X peak) per config, 1 GPU",
        "value": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(dtypes) + " (fp32 accumulate)" if len(dtypes) > 1 else dtypes[0],
        "data": "synthetic (seeded; x~N(0,1) or U[-1,1], w~N(0,1/fan_in), bias~U[-1,1]); inputs resident in HBM",
        "config": {"workload": " + ".join(inputs.WORKLOADS[n].about for n in names),
                   "names": names, "layout": "NHWGC/GKYXC -> NHWGK",
                   "step": "one gconv_fwd per listed workload (one kernel launch each)",
                   "cache": "hot (no rotation)" if a.hot else "rotating buffer sets >= 512 MB per workload"},
        "tflops": step_flops / (ms_per_step * 1e-3) / 1e12,
        "frac_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / metrics.PEAK_HBM_GBS,
        "per_config": per_config,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(names, a.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all", choices=sorted(WORKLOAD_SETS))
    ap.add_argument("--path", default="auto", help="force a kernel path (auto|generic|depthwise|smallg_mfma|igemm_mfma|ighalo_mfma)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=4, metavar="S",
                    help="bind an event pair to the dispatches of every S-th timed step (a dispatch-bound "
                         "event pair costs about 25 us of host time)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="rough bound on the CPU oracle's timing sample")
    ap.add_argument("--hot", action="store_true", help="no buffer rotation (cache-hot; labelled)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run 3 plain device copies of MIB MiB (a reference kernel of "
                         "known size for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--op", default="fwd", choices=["fwd", "bwd_data", "bwd_weight"],
                    help="bwd_data: time gconv_bwd_data (dx from dy and w); bwd_weight: gconv_bwd_weight "
                         "(dw from x and dy); both on the first workload of --workload")
    a = ap.parse_args()

    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        return 2

    import torch
    from depthwise_convolution_grouped_amd import gconv as G
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    G.lib()  # fail loudly if the HIP library is missing

    if a.calibrate_copy:
        nb = a.calibrate_copy << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if a.op == "bwd_data":
        return bench_bwd_data(a, G, torch)
    if a.op == "bwd_weight":
        return bench_bwd_weight(a, G, torch)
    return bench_fwd(a, G, torch)


if __name__ == "__main__":
    sys.exit(main())
