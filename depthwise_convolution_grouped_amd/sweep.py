"""Shape sweep: time every kernel path and every entry of its tile menu on
each shape, and compare the dispatcher's analytic choice (path and tile)
with the fastest.

    python -m depthwise_convolution_grouped_amd.sweep [--reps R] [--random N] [--out FILE]

This is the measured check of the analytic selection in gconv_host.cpp
(channels per group and dtype pick the path, each path's own scoring picks
its tile), the counterpart of the kernel enumeration and selection of the CK
grouped_conv tile engine (README: How It Works, Kernel Enumeration; the
Python examples README's ML heuristic), without a trained model: the
selection is a fixed rule, and this sweep measures how far it is from the
best (path, tile) on each shape.

Shapes: the benchmark workloads and variants around them (batch, channels
per group, stride, dilation, 3D), plus --random seeded random ones
(depthwise, small, medium and large groups; fp16, bf16, fp32; 2D and 3D;
strides, dilations, 1x1 / 3x3 / 5x5 windows).  Each (shape, path, tile) is
timed with an event pair around `reps` back-to-back launches, each on the
next of R rotating input / output buffer sets spanning >= 512 MB (twice the
256 MB Infinity Cache), inputs resident in HBM.  Prints one JSON line per
shape and, with --out, writes a Markdown summary.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

from depthwise_convolution_grouped_amd import inputs, metrics

ROTATE_BYTES = 512 << 20

# (name, problem): the workloads and variants around them
SHAPES = [
    ("depthwise s1 N=32 C=144 56^2 f16", inputs.conv2d("f16", 32, 144, 144, 144, 56, 56, 3, 3, 1, 1)),
    ("depthwise s2 N=32 C=144 56^2 f16", inputs.conv2d("f16", 32, 144, 144, 144, 56, 56, 3, 3, 2, 1)),
    ("depthwise s1 N=8 C=384 28^2 bf16", inputs.conv2d("bf16", 8, 384, 384, 384, 28, 28, 3, 3, 1, 1)),
    ("ResNeXt G=32 8/8 N=32 56^2 bf16", inputs.conv2d("bf16", 32, 32, 256, 256, 56, 56, 3, 3, 1, 1, bias=False)),
    ("ResNeXt G=32 16/16 N=16 28^2 bf16", inputs.conv2d("bf16", 16, 32, 512, 512, 28, 28, 3, 3, 1, 1, bias=False)),
    ("G=64 4/4 N=16 56^2 f16", inputs.conv2d("f16", 16, 64, 256, 256, 56, 56, 3, 3, 1, 1)),
    ("G=16 16/16 N=32 28^2 s2 bf16", inputs.conv2d("bf16", 32, 16, 256, 256, 28, 28, 3, 3, 2, 1)),
    ("3D G=32 2/4 N=8 8x28x28 f16", inputs.conv3d("f16", 8, 32, 64, 128, 8, 28, 28, 3, 3, 3, 1, 1)),
    ("3D G=32 2/4 N=1 8x28x28 f16", inputs.conv3d("f16", 1, 32, 64, 128, 8, 28, 28, 3, 3, 3, 1, 1)),
    ("G=8 128/128 N=64 14^2 bf16", inputs.conv2d("bf16", 64, 8, 1024, 1024, 14, 14, 3, 3, 1, 1)),
    ("G=8 128/128 N=64 14^2 dil2 bf16", inputs.conv2d("bf16", 64, 8, 1024, 1024, 14, 14, 3, 3, 1, 2, 2)),
    ("G=4 64/64 N=32 28^2 f16", inputs.conv2d("f16", 32, 4, 256, 256, 28, 28, 3, 3, 1, 1)),
    ("G=2 256/256 N=16 14^2 bf16", inputs.conv2d("bf16", 16, 2, 512, 512, 14, 14, 3, 3, 1, 1)),
    ("G=8 32/32 N=32 28^2 bf16", inputs.conv2d("bf16", 32, 8, 256, 256, 28, 28, 3, 3, 1, 1)),
    ("G=2 32/32 N=1 8^2 f32", inputs.conv2d("f32", 1, 2, 64, 64, 8, 8, 3, 3, 1, 1)),
    ("ResNeXt G=32 8/8 N=8 56^2 f32", inputs.conv2d("f32", 8, 32, 256, 256, 56, 56, 3, 3, 1, 1, bias=False)),
]


def random_shapes(n: int, seed: int = 2024):
    """Seeded random grouped/depthwise problems of 4..64 MB of input."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = str(rng.choice(["f16", "bf16", "f32"], p=[0.4, 0.4, 0.2]))
        ndim = 3 if rng.random() < 0.25 else 2
        kind = str(rng.choice(["depthwise", "small", "medium", "large"]))
        if kind == "depthwise":
            cpg = kpg = 1
            g = int(rng.choice([32, 64, 96, 144, 192, 240, 384, 576]))
        elif kind == "small":
            cpg = int(rng.choice([2, 4, 8, 16]))
            kpg = int(rng.choice([cpg, 2 * cpg]))
            g = int(rng.choice([8, 16, 32, 64]))
        elif kind == "medium":
            cpg = kpg = int(rng.choice([32, 64]))
            g = int(rng.choice([2, 4, 8]))
        else:
            cpg = kpg = int(rng.choice([128, 256]))
            g = int(rng.choice([1, 2, 4, 8]))
        k = int(rng.choice([1, 3, 3, 3, 5])) if ndim == 2 else 3
        stride = int(rng.choice([1, 1, 2]))
        dil = int(rng.choice([1, 1, 2])) if stride == 1 and k > 1 else 1
        pad = dil * (k - 1) // 2
        if ndim == 2:
            hw = int(rng.choice([7, 14, 28, 56, 112]))
            spatial = (1, hw, hw)
        else:
            hw = int(rng.choice([14, 28, 56]))
            spatial = (int(rng.choice([4, 8, 16])), hw, hw)
        es = 4 if dtype == "f32" else 2
        img = spatial[0] * spatial[1] * spatial[2] * g * cpg * es
        target = float(np.exp(rng.uniform(np.log(4e6), np.log(64e6))))
        N = max(1, min(256, int(target // img)))
        filt = (1, k, k) if ndim == 2 else (k, k, k)
        st = (1, stride, stride) if ndim == 2 else (stride,) * 3
        pd = (0, pad, pad) if ndim == 2 else (pad,) * 3
        dl = (1, dil, dil) if ndim == 2 else (dil,) * 3
        p = inputs.Problem(ndim, dtype, N, g, g * cpg, g * kpg, spatial, filt, st, pd, dl, bool(rng.random() < 0.5))
        if any(metrics.out_extent(spatial[a], filt[a], st[a], pd[a], dl[a]) < 1 for a in range(3)):
            continue
        name = "rand%02d %s %dD G=%d %d/%d N=%d %s k%d s%d d%d" % (
            len(out), kind, ndim, g, cpg, kpg, N, "x".join(str(v) for v in spatial[3 - ndim:]), k, stride, dil)
        out.append((name + " " + dtype, p))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--random", type=int, default=26, help="seeded random shapes added to the fixed ones")
    ap.add_argument("--seed", type=int, default=2024, help="seed of the random shapes")
    ap.add_argument("--random-only", action="store_true", help="the random shapes alone (a held-out set)")
    ap.add_argument("--dtype", default="", help="only the shapes of this element type (f16, bf16, f32)")
    ap.add_argument("--out", default="")
    a = ap.parse_args(argv)
    import torch
    from depthwise_convolution_grouped_amd import gconv as G
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    G.lib()
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    shapes = ([] if a.random_only else SHAPES) + random_shapes(a.random, a.seed)
    if a.dtype:
        shapes = [(n, p) for n, p in shapes if p.dtype == a.dtype]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    rows = []
    for name, p in shapes:
        d = G.desc_from_problem(p)
        o = G.gconv_out_dims(d)
        oshape = (p.N,) + (o if p.ndim == 3 else o[1:]) + (p.K,)
        per_set = metrics.io_bytes(p)["x"] + metrics.io_bytes(p)["y"]
        R = min(64, max(2, -(-ROTATE_BYTES // per_set)))
        gen = torch.Generator(device="cuda").manual_seed(1)
        x0 = torch.randn(p.x_shape(), device="cuda", generator=gen).to(tdt[p.dtype])
        xs = [x0] + [x0.clone() for _ in range(R - 1)]
        ys = [torch.empty(oshape, dtype=tdt[p.dtype], device="cuda") for _ in range(R)]
        w = (torch.randn(p.w_shape(), device="cuda", generator=gen) * 0.1).to(tdt[p.dtype])
        b = torch.randn((p.K,), device="cuda", generator=gen).to(tdt[p.dtype]) if p.bias else None
        bp = b.data_ptr() if b is not None else None

        def timed(pid, tile):
            for i in range(3):
                rc = G.gconv_fwd_tile(d, pid, tile, xs[i % R].data_ptr(), w.data_ptr(), bp, ys[i % R].data_ptr(), sp)
                if rc != 0:
                    raise G.GconvError(rc, "gconv_fwd_tile(%s)" % name)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(a.reps):
                G.gconv_fwd_tile(d, pid, tile, xs[i % R].data_ptr(), w.data_ptr(), bp, ys[i % R].data_ptr(), sp)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / a.reps * 1e3

        pick_path = G.gconv_path_name(G.gconv_select_path(d))
        times = {}
        own = {}
        for pname, pid in G.PATHS.items():
            if G.gconv_path_supported(d, pid) != 1:
                continue
            n, pk = G.gconv_tile_count(d, pid)
            own[pname] = pk
            # generic only with its own tile: its other menu entries are the
            # same kernel with other thread splits and take far longer
            tiles = [pk] if pname == "generic" and pname != pick_path else range(n)
            for t in tiles:
                times["%s/%d" % (pname, t)] = timed(pid, t)
        picked = "%s/%d" % (pick_path, own[pick_path])
        best = min(times, key=times.get)
        best_in_path = min((k for k in times if k.startswith(pick_path + "/")), key=times.get)
        r = {"shape": name, "picked": picked, "best": best, "best_in_path": best_in_path,
             "us": times, "picked_over_best": times[picked] / times[best],
             "picked_over_best_tile": times[picked] / times[best_in_path],
             "gbs_picked": metrics.total_bytes(p) / times[picked] / 1e3,
             "tflops_picked": metrics.flops(p) / times[picked] / 1e6, "rotating_sets": R}
        rows.append(r)
        print(json.dumps(r), flush=True)
        del xs, ys, w, b
        torch.cuda.empty_cache()
    within = sum(1 for r in rows if r["picked_over_best"] <= 1.05)
    path_right = sum(1 for r in rows if r["best"].split("/")[0] == r["picked"].split("/")[0])
    summary = {"shapes": len(rows), "picked_within_5pct_of_best": within,
               "picked_path_is_best_path": path_right,
               "median_picked_over_best": float(np.median([r["picked_over_best"] for r in rows])),
               "worst_picked_over_best": max(r["picked_over_best"] for r in rows)}
    print(json.dumps(summary), flush=True)
    if a.out:
        lines = ["| shape | picked (path/tile) | us | best | us | picked / best | best tile of the picked path | picked / that |",
                 "|---|---|---|---|---|---|---|---|"]
        for r in rows:
            lines.append("| %s | %s | %.1f | %s | %.1f | %.2f | %s | %.2f |" % (
                r["shape"], r["picked"], r["us"][r["picked"]], r["best"], r["us"][r["best"]],
                r["picked_over_best"], r["best_in_path"], r["picked_over_best_tile"]))
        lines += ["", "Summary: %d shapes; the pick is within 5%% of the best (path, tile) on %d (%.0f%%); "
                  "the picked path is the best path on %d; median picked / best %.3f, worst %.2f."
                  % (summary["shapes"], within, 100.0 * within / len(rows), path_right,
                     summary["median_picked_over_best"], summary["worst_picked_over_best"])]
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
