"""Shape sweep: time every kernel path that can run each shape and compare
the dispatcher's analytic choice with the fastest.

    python -m depthwise_convolution_grouped_amd.sweep [--reps R] [--out FILE]

This is the measured check of the analytic path and tile selection in
gconv_host.cpp (channels per group, dtype, then each path's own tile
scoring), the counterpart of the kernel enumeration and selection of the CK
grouped_conv tile engine (Kernel Enumeration; ML heuristic), without a
trained model: the selection is a fixed rule, and this sweep measures how
far it is from the best path on each shape.

Each (shape, path) is timed with an event pair around `reps` back-to-back
launches on the current stream, inputs resident in HBM and reused (a hot
cache, so absolute times are lower than bench.py's rotating-buffer ones;
the comparison between paths is what the sweep is for).  Prints one line
per shape and, with --out, writes a Markdown table.
"""
from __future__ import annotations

import argparse
import json
import sys

from depthwise_convolution_grouped_amd import inputs, metrics

# (name, problem): the workloads and variants around them (batch, channels
# per group, stride, dilation, 3D)
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
]


def time_path(G, torch, d, path, x, w, b, y, reps):
    s = torch.cuda.current_stream()
    sp = s.cuda_stream
    for _ in range(3):
        rc = G.gconv_fwd_path(d, path, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                              y.data_ptr(), sp)
        if rc != 0:
            raise G.GconvError(rc, "gconv_fwd_path")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        G.gconv_fwd_path(d, path, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                         y.data_ptr(), sp)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--out", default="")
    a = ap.parse_args(argv)
    import torch
    from depthwise_convolution_grouped_amd import gconv as G
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    G.lib()
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    rows = []
    for name, p in SHAPES:
        d = G.desc_from_problem(p)
        o = G.gconv_out_dims(d)
        gen = torch.Generator(device="cuda").manual_seed(1)
        x = torch.randn(p.x_shape(), device="cuda", generator=gen).to(tdt[p.dtype])
        w = torch.randn(p.w_shape(), device="cuda", generator=gen).to(tdt[p.dtype])
        b = torch.randn((p.K,), device="cuda", generator=gen).to(tdt[p.dtype]) if p.bias else None
        y = torch.empty((p.N,) + (o if p.ndim == 3 else o[1:]) + (p.K,), dtype=tdt[p.dtype], device="cuda")
        picked = G.gconv_path_name(G.gconv_select_path(d))
        times = {}
        for pname, pid in G.PATHS.items():
            if G.gconv_path_supported(d, pid) == 1:
                times[pname] = time_path(G, torch, d, pid, x, w, b, y, a.reps)
        best = min(times, key=times.get)
        r = {"shape": name, "picked": picked, "best": best, "us": times,
             "picked_over_best": times[picked] / times[best],
             "gbs_picked": metrics.total_bytes(p) / times[picked] / 1e3,
             "tflops_picked": metrics.flops(p) / times[picked] / 1e6}
        rows.append(r)
        print(json.dumps(r), flush=True)
        del x, w, b, y
    if a.out:
        names = list(G.PATHS)
        lines = ["| shape | picked | best | picked / best | " + " | ".join(names) + " |",
                 "|---|---|---|---|" + "---|" * len(names)]
        for r in rows:
            cells = ["%.1f" % r["us"][n] if n in r["us"] else "-" for n in names]
            lines.append("| %s | %s | %s | %.2f | %s |" % (r["shape"], r["picked"], r["best"],
                                                          r["picked_over_best"], " | ".join(cells)))
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
