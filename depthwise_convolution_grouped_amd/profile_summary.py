"""Summarise rocprofv3 output for one workload into profiles/.

    python -m depthwise_convolution_grouped_amd.profile_summary \\
        --workload depthwise2d_f16 --trace DIR [--fetch DIR --write DIR] \\
        --trace-cmd "..." [--pmc-cmd "..."]

--trace  a `rocprofv3 --kernel-trace --stats -f csv` output directory
--fetch  a `rocprofv3 --pmc FETCH_SIZE -f csv` directory of a bench.py run
         with --calibrate-copy MIB (a plain copy kernel of known size)
--write  the same with WRITE_SIZE
--counters DIR [DIR ...]  `rocprofv3 --pmc ...` directories of bench.py runs
         (one per counter pass), with --counter-cmds giving each pass's command

Writes profiles/<kernel>__<workload>.md (kernel durations; HBM bytes per
launch from the counters, each scaled by what the same counter reads for the
reference copy) and updates profiles/traffic.json, which bench.py reads back
as the roofline's `traffic` while the kernel sources are unchanged.  With
--counters it also writes profiles/counters__<kernel>__<workload>.md: the
per-dispatch medians of every counter collected for the kernel and the
figures derived from them (matrix-core issue against the FLOPs the problem
needs, matrix pipe and texture-address busy fractions over the traced kernel
time at the 2.4 GHz peak clock, LDS bank-conflict share, L2 read latency).
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


N_SIMD, N_CU, CLOCK_MHZ = 1024, 256, 2400.0     # MI355X: 256 CUs x 4 SIMDs, 2.4 GHz peak
MFMA_FLOP, MFMA_CYCLES = 16 * 16 * 32 * 2, 16     # one v_mfma_f32_16x16x32 (bf16 / fp16)


def counter_medians(dirs, kernel_name, grid_items):
    """{counter: median per dispatch} for our kernel over the given pmc runs."""
    out = {}
    for d in dirs:
        vals = {}
        for r in _rows(d, "*counter_collection.csv"):
            if r["Kernel_Name"] == kernel_name and int(r["Grid_Size"]) == grid_items:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for c, v in vals.items():
            out[c] = statistics.median(v)
    return out


def counters_page(path, workload, about, kernel_name, med_us, flop, cm, cmds):
    lines = ["# Counters of the %s kernel on %s" % (path, workload), "",
             "Workload: %s." % about, "", "Kernel: `%s`" % kernel_name[:160], "",
             "Commands (one counter pass each; counters per pass within the hardware's block limits):", ""]
    lines += ["    " + c for c in cmds]
    lines += ["", "Per-dispatch medians (sums over the whole GPU):", "", "| counter | value |", "|---|---|"]
    for c in sorted(cm):
        lines.append("| %s | %.6g |" % (c, cm[c]))
    cyc = med_us * CLOCK_MHZ
    lines += ["", "Derived, with the kernel's median traced duration of %.2f us (%.0f cycles at 2.4 GHz):" % (med_us, cyc), ""]
    if cm.get("SQ_INSTS_MFMA"):
        need = flop / MFMA_FLOP
        lines.append("- MFMA instructions: %.0f issued, %.0f needed by the problem's FLOPs: %.3f x."
                     % (cm["SQ_INSTS_MFMA"], need, cm["SQ_INSTS_MFMA"] / need))
        busy = cm.get("SQ_VALU_MFMA_BUSY_CYCLES", cm["SQ_INSTS_MFMA"] * MFMA_CYCLES)
        lines.append("- matrix pipes busy %.1f%% of the kernel time (SQ_VALU_MFMA_BUSY_CYCLES over %d SIMDs); "
                     "the useful part (needed MFMAs) is %.1f%%."
                     % (100.0 * busy / (N_SIMD * cyc), N_SIMD, 100.0 * need * MFMA_CYCLES / (N_SIMD * cyc)))
    if cm.get("SQ_LDS_IDX_ACTIVE"):
        lines.append("- LDS: bank-conflict cycles are %.1f%% of the LDS-active cycles; LDS active %.1f%% of "
                     "the kernel time per CU." % (100.0 * cm.get("SQ_LDS_BANK_CONFLICT", 0.0) / cm["SQ_LDS_IDX_ACTIVE"],
                                                   100.0 * cm["SQ_LDS_IDX_ACTIVE"] / (N_CU * cyc)))
    if cm.get("TA_TA_BUSY_sum"):
        lines.append("- texture address unit busy %.1f%% of the kernel time (TA_TA_BUSY over %d CUs), %.1f%% of "
                     "that stalled by the L1 (TA_ADDR_STALLED_BY_TC_CYCLES)."
                     % (100.0 * cm["TA_TA_BUSY_sum"] / (N_CU * cyc), N_CU,
                        100.0 * cm.get("TA_ADDR_STALLED_BY_TC_CYCLES_sum", 0.0) / cm["TA_TA_BUSY_sum"]))
    if cm.get("TCP_TCC_READ_REQ_sum"):
        lines.append("- L1 -> L2 reads: %.0f requests, %.0f cycles average latency."
                     % (cm["TCP_TCC_READ_REQ_sum"], cm.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / cm["TCP_TCC_READ_REQ_sum"]))
    if cm.get("SQ_WAVES"):
        per = lambda k: cm.get(k, 0.0) / cm["SQ_WAVES"]
        lines.append("- per wave: %.0f VALU, %.0f MFMA, %.0f LDS, %.0f vector-memory read and %.0f write instructions."
                     % (per("SQ_INSTS_VALU"), per("SQ_INSTS_MFMA"), per("SQ_INSTS_LDS"),
                        per("SQ_INSTS_VMEM_RD"), per("SQ_INSTS_VMEM_WR")))
    return lines


def backward_page(a, p, inputs, metrics):
    """profiles/<op>__<workload>.md for a backward call (every kernel it
    launches, each once per call) and its traffic.json entry."""
    alg_bytes, alg_flop = metrics.total_bytes(p), metrics.flops(p)
    stats = [r for r in _rows(a.trace, "*kernel_stats.csv") if "gconv" in r["Name"]]
    what = {"bwd_data": "backward data (dx from dy and w)", "bwd_weight": "backward weight (dw from x and dy)"}[a.op]
    lines = ["# %s on %s" % (what.split(" (")[0], a.workload), "",
             "Workload: %s; %s." % (inputs.WORKLOADS[a.workload].about, what), "",
             "Algorithmic work per call: %d FLOP, %d bytes (each tensor once)." % (alg_flop, alg_bytes), "",
             "## Kernel trace", "", "Command:", "", "    " + a.trace_cmd, "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    tot = 0.0
    for r in stats:
        avg = float(r["AverageNs"]) / 1e3
        tot += avg
        lines.append("| %s | %s | %.2f | %.2f | %.2f |" % (r["Name"][:90], r["Calls"], avg,
                                                           float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    lines += ["", "Kernel time per call (each kernel runs once per call): %.2f us -> %.1f GB/s, %.2f TFLOP/s "
              "(algorithmic)." % (tot, alg_bytes / tot / 1e3, alg_flop / tot / 1e6)]
    entry = None
    if a.fetch and a.write:
        def per_call(d, counter):
            ours, copies = {}, []
            for r in _rows(d, "*counter_collection.csv"):
                if r["Counter_Name"] != counter:
                    continue
                if "copyBuffer" in r["Kernel_Name"]:
                    copies.append(float(r["Counter_Value"]))
                elif "gconv" in r["Kernel_Name"]:
                    ours.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            return sum(statistics.median(v) for v in ours.values()), max(copies)
        f_kib, f_ref = per_call(a.fetch, "FETCH_SIZE")
        w_kib, w_ref = per_call(a.write, "WRITE_SIZE")
        ref_kib = a.copy_mib * 1024.0
        f_scale, w_scale = ref_kib / f_ref, ref_kib / w_ref
        hbm = f_kib * 1024 * f_scale + w_kib * 1024 * w_scale
        lines += ["", "## HBM traffic (rocprofv3 counters)", "", "Commands (one counter per run):", "",
                  "    " + a.pmc_cmd.replace("COUNTER", "FETCH_SIZE"),
                  "    " + a.pmc_cmd.replace("COUNTER", "WRITE_SIZE"), "",
                  "A %d MiB device copy reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB, so the "
                  "counters are scaled by %.3f and %.3f." % (a.copy_mib, f_ref, w_ref, f_scale, w_scale), "",
                  "| counter | KiB per call (sum of the kernels' per-dispatch medians) | scaled bytes |",
                  "|---|---|---|",
                  "| FETCH_SIZE | %.0f | %.0f |" % (f_kib, f_kib * 1024 * f_scale),
                  "| WRITE_SIZE | %.0f | %.0f |" % (w_kib, w_kib * 1024 * w_scale), "",
                  "HBM bytes per call: %.0f = %.3f x the algorithmic %d." % (hbm, hbm / alg_bytes, alg_bytes)]
        entry = {"kernel": a.op, "source_hash": source_hash(a.op), "hbm_bytes_per_launch": hbm,
                 "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": f_scale,
                 "write_scale": w_scale, "algorithmic_bytes": alg_bytes}
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "%s__%s.md" % (a.op, a.workload))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)
    if entry:
        try:
            with open(TRAFFIC) as f:
                db = json.load(f)
        except (OSError, ValueError):
            db = {}
        db["%s:%s" % (a.op, a.workload)] = entry
        with open(TRAFFIC, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)
        print("updated", TRAFFIC)


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
    ap.add_argument("--counters", nargs="*", default=[])
    ap.add_argument("--counter-cmds", nargs="*", default=[])
    ap.add_argument("--op", default="fwd", choices=["fwd", "bwd_data", "bwd_weight"])
    a = ap.parse_args(argv)

    p = inputs.WORKLOADS[a.workload].problem
    if a.op != "fwd":
        return backward_page(a, p, inputs, metrics)
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
    if a.counters:
        cm = counter_medians(a.counters, kernel_name, grid_items)
        page = counters_page(path, a.workload, inputs.WORKLOADS[a.workload].about, kernel_name,
                             statistics.median(durs), alg_flop, cm, a.counter_cmds)
        cout = os.path.join(PROFILES, "counters__%s__%s.md" % (path, a.workload))
        with open(cout, "w") as f:
            f.write("\n".join(page) + "\n")
        print("wrote", cout)
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
