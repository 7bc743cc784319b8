"""Summarise rocprofv3 output for one workload into profiles/.

    python -m depthwise_convolution_grouped_amd.profile_summary \\
        --workload depthwise2d_f16 --trace DIR [--fetch DIR --write DIR] \\
        --trace-cmd "..." [--pmc-cmd "..."]

--trace  a `rocprofv3 --kernel-trace --stats -f csv` output directory
--fetch  a `rocprofv3 --pmc FETCH_SIZE -f csv` directory of a bench.py run
         with --calibrate-copy MIB (a plain copy kernel of known size)
--write  the same with WRITE_SIZE

Writes profiles/<kernel>__<workload>.md (kernel durations; HBM bytes per
launch from the counters, each scaled by what the same counter reads for the
reference copy) and updates profiles/traffic.json, which bench.py reads back
as the roofline's `traffic` while the kernel sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC = os.path.join(PROFILES, "traffic.json")

# kernel path name -> source file whose text (with the shared headers) the counters belong to
PATH_SOURCES = {
    "generic": "k_generic.hip",
    "depthwise": "k_depthwise.hip",
    "smallg_mfma": ("k_smallg.hip", "k_smallg_rows.hip", "k_smallg_ring.hip", "k_smallg_ring3d.hip",
                    "smallg_common.h", "smallg_ring.h"),
    "igemm_mfma": "k_igemm.hip",
    "ighalo_mfma": ("k_ighalo.hip", "k_ighalo_box.hip"),
    "direct_valu": "k_direct.hip",
}
SHARED = ("device_common.h", "gconv_internal.h")
KERNEL_TAGS = {"generic": "generic", "depthwise": "depthwise", "smallg_mfma": "smallg",
               "igemm_mfma": "igemm", "ighalo_mfma": "ighalo", "direct_valu": "direct"}


def source_hash(path_name: str) -> str:
    """Hash of the sources a path's kernels are built from.  The backward
    routes run forward kernels too, so every kernel source counts for them."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    if path_name in ("bwd_data", "bwd_weight"):
        files = tuple(sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))))
    else:
        own = PATH_SOURCES[path_name]
        files = (own if isinstance(own, tuple) else (own,)) + SHARED
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _rows(d, name):
    files = glob.glob(os.path.join(d, "**", name), recursive=True)
    if not files:
        raise SystemExit("no %s under %s" % (name, d))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(d, counter, kernel_name, grid_items):
    """(values for dispatches of our kernel, values for the calibration copies).

    Our kernel is the exact symbol picked from the trace, with our grid size
    in work-items (other configs of a workload may run another instance of
    the same template, or the same instance on another grid)."""
    ours, copies = [], []
    for r in _rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if name == kernel_name and int(r["Grid_Size"]) == grid_items:
            ours.append(v)
        elif "copyBuffer" in name:
            copies.append(v)
    return ours, copies


def main(argv=None):
    import sys
    sys.path.insert(0, ROOT)
    from depthwise_convolution_grouped_amd import inputs, metrics
    from depthwise_convolution_grouped_amd import gconv as G

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-mib", type=int, default=64)
    ap.add_argument("--trace-cmd", required=True)
    ap.add_argument("--pmc-cmd", default="")
    a = ap.parse_args(argv)

    p = inputs.WORKLOADS[a.workload].problem
    d = G.desc_from_problem(p)
    path = G.gconv_path_name(G.gconv_select_path(d))
    tag = KERNEL_TAGS[path]
    alg_bytes = metrics.total_bytes(p)
    alg_flop = metrics.flops(p)
    plan = G.gconv_get_plan(d)
    grid_items = plan["grid"][0] * plan["grid"][1] * plan["grid"][2] * plan["block"]

    stats = [r for r in _rows(a.trace, "*kernel_stats.csv") if "gconv" in r["Name"]]
    trace = [r for r in _rows(a.trace, "*kernel_trace.csv")
             if "gconv" in r["Kernel_Name"] and tag in r["Kernel_Name"] and
             int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) == grid_items]
    grids = "%s x %d threads" % (tuple(plan["grid"]), plan["block"])
    if not trace:
        raise SystemExit("no dispatch of the %s kernel with %d work-items in %s" % (path, grid_items, a.trace))
    # several template instances of the path can share the grid (a workload's
    # second config): ours is the one with the most kernel time
    total = {}
    for r in trace:
        total[r["Kernel_Name"]] = total.get(r["Kernel_Name"], 0) + int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    kernel_name = max(total, key=total.get)
    trace = [r for r in trace if r["Kernel_Name"] == kernel_name]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in trace]
    lines = ["# %s kernel on %s" % (path, a.workload), "",
             "Workload: %s." % inputs.WORKLOADS[a.workload].about, "",
             "Algorithmic work per launch: %d FLOP, %d bytes (x, w, bias and y once each)."
             % (alg_flop, alg_bytes), "",
             "## Kernel trace", "", "Command:", "", "    " + a.trace_cmd, "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append("| %s | %s | %.2f | %.2f | %.2f |" % (
            r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    if durs:
        med = statistics.median(durs)
        lines += ["", "Dispatches of the %s kernel: %d, median %.2f us -> %.1f GB/s, %.2f TFLOP/s "
                  "(algorithmic); grid %s." % (path, len(durs), med, alg_bytes / med / 1e3,
                                              alg_flop / med / 1e6, grids)]
    entry = None
    if a.fetch and a.write:
        f_ours, f_copy = counter_per_dispatch(a.fetch, "FETCH_SIZE", kernel_name, grid_items)
        w_ours, w_copy = counter_per_dispatch(a.write, "WRITE_SIZE", kernel_name, grid_items)
        ref_kib = a.copy_mib * 1024.0
        # the calibration copies are the largest copyBuffer dispatches (MIB MiB each)
        f_ref = max(f_copy) if f_copy else None
        w_ref = max(w_copy) if w_copy else None
        f_scale = ref_kib / f_ref if f_ref else None
        w_scale = ref_kib / w_ref if w_ref else None
        f_kib = statistics.median(f_ours)
        w_kib = statistics.median(w_ours)
        hbm = f_kib * 1024 * f_scale + w_kib * 1024 * w_scale
        lines += ["", "## HBM traffic (rocprofv3 counters)", "", "Commands (one counter per run):", "",
                  "    " + a.pmc_cmd.replace("COUNTER", "FETCH_SIZE"),
                  "    " + a.pmc_cmd.replace("COUNTER", "WRITE_SIZE"), "",
                  "A %d MiB device copy reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB, so the "
                  "counters are scaled by %.3f and %.3f." % (a.copy_mib, f_ref, w_ref, f_scale, w_scale), "",
                  "| counter | KiB per dispatch (median) | scaled bytes |", "|---|---|---|",
                  "| FETCH_SIZE | %.0f | %.0f |" % (f_kib, f_kib * 1024 * f_scale),
                  "| WRITE_SIZE | %.0f | %.0f |" % (w_kib, w_kib * 1024 * w_scale), "",
                  "HBM bytes per launch: %.0f = %.3f x the algorithmic %d." % (hbm, hbm / alg_bytes, alg_bytes)]
        entry = {"kernel": path, "source_hash": source_hash(path), "hbm_bytes_per_launch": hbm,
                 "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": f_scale,
                 "write_scale": w_scale, "algorithmic_bytes": alg_bytes}
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "%s__%s.md" % (path, a.workload))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)
    if entry:
        try:
            with open(TRAFFIC) as f:
                db = json.load(f)
        except (OSError, ValueError):
            db = {}
        db[a.workload] = entry
        with open(TRAFFIC, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)
        print("updated", TRAFFIC)


if __name__ == "__main__":
    main()
