"""Work accounting for grouped conv forward: algorithmic FLOP and HBM bytes.

Conventions of the TileOPs PR 1568 review (section "The 50x is a baseline
artifact"): FLOP = outputs x MACs per output x 2, where MACs per output count
every tap of the window (padded taps included) times the input channels of
ONE group (per-group C_in, as the same review's manifest note demands); bytes
count the input, the output and the weights once each, plus the bias when
present.
"""
from __future__ import annotations

from .inputs import Problem, element_size

# MI355X published peaks (dense; not the sparsity figures).
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32_vector": 157.3, "f32_mfma": 157.3}


def out_extent(n: int, k: int, s: int, p: int, d: int) -> int:
    room = n + 2 * p - (d * (k - 1) + 1)
    return room // s + 1 if room >= 0 else 0


def out_spatial(p: Problem):
    return tuple(out_extent(p.spatial[a], p.filt[a], p.stride[a], p.pad[a], p.dil[a])
                 for a in range(3))


def outputs(p: Problem) -> int:
    Do, Ho, Wo = out_spatial(p)
    return p.N * Do * Ho * Wo * p.K


def macs_per_output(p: Problem) -> int:
    return p.Cpg * p.filt[0] * p.filt[1] * p.filt[2]


def flops(p: Problem) -> int:
    return 2 * outputs(p) * macs_per_output(p)


def io_bytes(p: Problem) -> dict:
    e = element_size(p.dtype)
    D, H, W = p.spatial
    return {
        "x": e * p.N * D * H * W * p.C,
        "y": e * outputs(p),
        "w": e * p.K * macs_per_output(p),
        "bias": e * p.K if p.bias else 0,
    }


def total_bytes(p: Problem) -> int:
    return sum(io_bytes(p).values())


def rates(p: Problem, seconds: float) -> dict:
    """TFLOP/s, GB/s and both as fractions of the MI355X peaks for one call of `seconds`."""
    tf = flops(p) / seconds / 1e12
    gbs = total_bytes(p) / seconds / 1e9
    peak_tf = PEAK_TFLOPS["f32_vector"] if p.dtype == "f32" else PEAK_TFLOPS[p.dtype]
    return {"tflops": tf, "gbs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
            "frac_compute": tf / peak_tf, "arith_intensity": flops(p) / total_bytes(p)}
