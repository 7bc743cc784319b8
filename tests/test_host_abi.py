"""Host side of the C ABI, without a GPU: exports, validation, extents,
path selection and launch plans.  Nothing here launches a kernel: every call
either is a pure host function or fails validation before a launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from depthwise_convolution_grouped_amd import gconv as G
from depthwise_convolution_grouped_amd import inputs, metrics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gconv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gconv_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 10, names
    L = G.lib()
    for n in names:
        assert hasattr(L, n), "libgconv.so does not export %s" % n
    assert set(names) == set(G.EXPORTS)


def test_exports_nothing_else():
    import subprocess
    r = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("nm unavailable")
    syms = {line.split()[-1] for line in r.stdout.splitlines() if line.strip()}
    ours = {s for s in syms if s.startswith("gconv")}
    assert ours == set(declared_functions())
    assert not any(s.startswith("_ZN5gconv") for s in syms), "internal C++ symbols leak"


def test_abi_version():
    assert G.gconv_abi_version() == 1


def base_desc(**kw):
    a = dict(ndim=2, dtype="f16", N=2, G=4, C=8, K=12, spatial=(9, 10), filt=(3, 3),
             stride=(1, 1), pad=(1, 1), dil=(1, 1))
    a.update(kw)
    return G.make_desc(**a)


def test_valid_descriptor():
    assert G.gconv_validate(base_desc()) == G.GCONV_OK


@pytest.mark.parametrize("kw,status", [
    (dict(ndim=4), G.GCONV_ERR_BAD_DESC),
    (dict(ndim=1), G.GCONV_ERR_BAD_DESC),
    (dict(dtype=7), G.GCONV_ERR_BAD_DESC),
    (dict(C=9), G.GCONV_ERR_BAD_DESC),            # C % G != 0
    (dict(K=10), G.GCONV_ERR_BAD_DESC),           # K % G != 0
    (dict(N=0), G.GCONV_ERR_BAD_DESC),
    (dict(G=0), G.GCONV_ERR_BAD_DESC),
    (dict(stride=(0, 1)), G.GCONV_ERR_BAD_DESC),
    (dict(dil=(1, 0)), G.GCONV_ERR_BAD_DESC),
    (dict(pad=(-1, 0)), G.GCONV_ERR_BAD_DESC),
    (dict(spatial=(0, 4)), G.GCONV_ERR_BAD_DESC),
    (dict(filt=(3, 0)), G.GCONV_ERR_BAD_DESC),
    (dict(spatial=(2, 2), pad=(0, 0)), G.GCONV_ERR_BAD_OUT_DIMS),
    (dict(spatial=(5, 5), pad=(0, 0), dil=(3, 3)), G.GCONV_ERR_BAD_OUT_DIMS),
    (dict(N=1 << 20, spatial=(1024, 1024)), G.GCONV_OK),           # split into launches of whole images
    (dict(N=1, spatial=(65536, 65536)), G.GCONV_OK),               # one image of 2^35 elements: split into row slices
    (dict(N=1, spatial=(4, 1 << 28)), G.GCONV_ERR_TOO_LARGE),      # one row of x spans 2^32 bytes: no slice fits
    (dict(N=1 << 40), G.GCONV_ERR_TOO_LARGE),
])
def test_validation_errors(kw, status):
    assert G.gconv_validate(base_desc(**kw)) == status


def test_2d_with_depth_entries_is_rejected():
    d = base_desc()
    d.in_[0] = 2
    assert G.gconv_validate(d) == G.GCONV_ERR_BAD_DESC
    d = base_desc()
    d.pad[0] = 1
    assert G.gconv_validate(d) == G.GCONV_ERR_BAD_DESC


def test_null_descriptor():
    L = G.lib()
    assert L.gconv_validate(None) == G.GCONV_ERR_NULL_PTR
    assert L.gconv_select_path(None) == G.GCONV_ERR_NULL_PTR


def test_out_dims_match_metrics_random():
    rng = np.random.default_rng(5)
    for i in range(300):
        p = inputs.random_problem(rng, ["f32", "f16", "bf16"][i % 3], 2 + i % 2)
        d = G.desc_from_problem(p)
        assert G.gconv_validate(d) == G.GCONV_OK
        assert G.gconv_out_dims(d) == metrics.out_spatial(p)


def test_out_dims_match_oracle_on_workloads():
    import oracle
    for name, wl in inputs.WORKLOADS.items():
        p = wl.problem
        o = G.gconv_out_dims(G.desc_from_problem(p))
        for a in range(3):
            assert o[a] == oracle.out_extent(p.spatial[a], p.filt[a], p.stride[a], p.pad[a], p.dil[a]), name


# Paths the dispatcher must pick for the workloads (channels per group decide).
EXPECTED_PATH = {
    "grouped2d_small_f32": "generic",
    "depthwise2d_f16": "depthwise",
    "depthwise2d_s2_f16": "depthwise",
    "grouped2d_resnext_bf16": "smallg_mfma",
    "grouped3d_f16_n1": "smallg_mfma",
    "grouped3d_f16_n8": "smallg_mfma",
    "grouped2d_large_bf16": "ighalo_mfma",
    "grouped2d_large_dil2_bf16": "ighalo_mfma",
}


def _built_paths():
    d = G.desc_from_problem(inputs.WORKLOADS["depthwise2d_f16"].problem)
    out = {"generic"}
    for name, pid in G.PATHS.items():
        probe = {"depthwise": "depthwise2d_f16", "smallg_mfma": "grouped2d_resnext_bf16",
                 "igemm_mfma": "grouped2d_large_bf16", "ighalo_mfma": "grouped2d_large_bf16",
                 "direct_valu": "grouped2d_small_f32", "generic": "depthwise2d_f16"}[name]
        d = G.desc_from_problem(inputs.WORKLOADS[probe].problem)
        if G.gconv_path_supported(d, pid) == 1:
            out.add(name)
    return out


@pytest.mark.parametrize("name", sorted(EXPECTED_PATH))
def test_dispatch_per_workload(name):
    want = EXPECTED_PATH[name]
    if want not in _built_paths():
        pytest.skip("path %s not built" % want)
    d = G.desc_from_problem(inputs.WORKLOADS[name].problem)
    assert G.gconv_path_name(G.gconv_select_path(d)) == want


def test_generic_supports_everything_and_plans():
    rng = np.random.default_rng(9)
    for i in range(100):
        p = inputs.random_problem(rng, "f16", 2 + i % 2)
        d = G.desc_from_problem(p)
        assert G.gconv_path_supported(d, G.GCONV_PATH_GENERIC) == 1
        pl = G.gconv_get_plan(d, G.GCONV_PATH_GENERIC)
        assert pl["grid"][0] * pl["block"] >= metrics.outputs(p)
        sel = G.gconv_select_path(d)
        assert 0 <= sel < G.GCONV_NUM_PATHS
        assert G.gconv_path_supported(d, sel) == 1
        assert G.gconv_get_plan(d)["path"] == sel


def test_bad_path_ids():
    d = base_desc()
    assert G.gconv_path_supported(d, 17) == G.GCONV_ERR_BAD_PATH
    with pytest.raises(G.GconvError):
        G.gconv_get_plan(d, 17)


def test_errors_return_before_launch():
    d = base_desc()
    # null x / w / y
    assert G.gconv_fwd(d, 0, 256, None, 512) == G.GCONV_ERR_NULL_PTR
    assert G.gconv_fwd(d, 256, 0, None, 512) == G.GCONV_ERR_NULL_PTR
    assert G.gconv_fwd(d, 256, 256, None, 0) == G.GCONV_ERR_NULL_PTR
    # element misalignment (fp16 needs 2-byte alignment)
    assert G.gconv_fwd(d, 257, 256, None, 512) == G.GCONV_ERR_MISALIGNED
    assert G.gconv_fwd(d, 256, 256, 259, 512) == G.GCONV_ERR_MISALIGNED
    # bad descriptor wins over pointers
    assert G.gconv_fwd(base_desc(C=9), 256, 256, None, 512) == G.GCONV_ERR_BAD_DESC
    # unknown path id
    assert G.gconv_fwd_path(d, 9, 256, 256, None, 512) == G.GCONV_ERR_BAD_PATH


def test_forced_vector_path_needs_16_byte_alignment():
    for name, pid in G.PATHS.items():
        if name == "generic" or name not in _built_paths():
            continue
        probe = {"depthwise": "depthwise2d_f16", "smallg_mfma": "grouped2d_resnext_bf16",
                 "igemm_mfma": "grouped2d_large_bf16", "ighalo_mfma": "grouped2d_large_bf16",
                 "direct_valu": "grouped2d_small_f32"}[name]
        d = G.desc_from_problem(inputs.WORKLOADS[probe].problem)
        assert G.gconv_fwd_path(d, pid, 256 + 2, 256, None, 512) == G.GCONV_ERR_MISALIGNED
        # bias is read in 16-byte vectors too
        assert G.gconv_fwd_path(d, pid, 256, 256, 256 + 2, 512) == G.GCONV_ERR_MISALIGNED
        assert G.gconv_fwd_path(d, pid, 256, 256, 256 + 8, 512) == G.GCONV_ERR_MISALIGNED


def test_forced_unsupported_path():
    # fp32 grouped problem with 3 channels per group: no MFMA path takes it
    d = G.make_desc(2, "f32", 1, 2, 6, 6, (8, 8), (3, 3), (1, 1), (1, 1), (1, 1))
    for pid in (G.GCONV_PATH_DEPTHWISE, G.GCONV_PATH_SMALLG, G.GCONV_PATH_IGEMM,
                G.GCONV_PATH_IGHALO):
        assert G.gconv_path_supported(d, pid) == 0
        assert G.gconv_fwd_path(d, pid, 256, 256, None, 512) == G.GCONV_ERR_PATH_UNSUPPORTED


def test_status_strings():
    for s in range(-9, 1):
        assert isinstance(G.gconv_status_str(s), str) and G.gconv_status_str(s)
    assert G.gconv_path_name(G.GCONV_PATH_AUTO) == "auto"
    assert [G.gconv_path_name(i) for i in range(G.GCONV_NUM_PATHS)] == list(G.PATHS)


def test_bwd_data_workspace_sizes():
    # stride 1 with dil (k - 1) >= pad: the transform route needs a copy of w
    d = G.make_desc(2, "bf16", 2, 4, 64, 32, (9, 9), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_bwd_data_workspace(d) == 32 * 3 * 3 * 16 * 2
    d = G.make_desc(3, "f32", 1, 2, 4, 6, (5, 6, 7), (3, 1, 3), (1, 1, 1), (1, 0, 2), (1, 1, 1))
    assert G.gconv_bwd_data_workspace(d) == 6 * 3 * 1 * 3 * 2 * 4
    # stride 2, groups other than depthwise: the residue classes' reversed
    # sub-kernels (1x1, 1x2, 2x1, 2x2 of 8 x 8 channels, each rounded to 256
    # bytes) and a dense buffer for the largest class (5 x 5 pixels of 8)
    d = G.make_desc(2, "f16", 1, 1, 8, 8, (9, 9), (3, 3), (2, 2), (1, 1), (1, 1))
    assert G.gconv_bwd_data_workspace(d) == 256 + 256 + 256 + 512 + 512
    # depthwise at stride 2 runs its channel-vector direct kernel, at stride 1
    # the forward depthwise kernel with each window reversed (no weight
    # copy), and a pad beyond the dilated filter has no use for one
    d = G.make_desc(2, "f16", 1, 16, 16, 16, (9, 9), (3, 3), (2, 2), (1, 1), (1, 1))
    assert G.gconv_bwd_data_workspace(d) == 0
    d = G.make_desc(2, "f16", 1, 16, 16, 16, (9, 9), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_bwd_data_workspace(d) == 0
    d = G.make_desc(2, "f16", 1, 1, 8, 8, (9, 9), (3, 3), (1, 1), (3, 3), (1, 1))
    assert G.gconv_bwd_data_workspace(d) == 0


def test_bwd_data_validates_before_any_launch():
    bad = G.make_desc(2, "f16", 1, 3, 8, 8, (9, 9), (3, 3), (1, 1), (1, 1), (1, 1))   # C % G != 0
    with pytest.raises(G.GconvError):
        G.gconv_bwd_data_workspace(bad)
    assert G.gconv_bwd_data(bad, 16, 16, 16, None, 0) == G.GCONV_ERR_BAD_DESC
    ok = G.make_desc(2, "f16", 1, 1, 8, 8, (9, 9), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_bwd_data(ok, 0, 16, 16, None, 0) == G.GCONV_ERR_NULL_PTR
    assert G.gconv_bwd_data_direct(ok, 16, 16, 0) == G.GCONV_ERR_NULL_PTR
    assert G.gconv_bwd_data(ok, 17, 16, 16, None, 0) == G.GCONV_ERR_MISALIGNED


def test_bwd_weight_workspace_and_validation():
    # depthwise 3x3 (channel-vector route): up to 512 chunks of G * 9 fp32 partial sums
    d = G.make_desc(2, "f16", 2, 16, 16, 16, (13, 17), (3, 3), (1, 1), (1, 1), (1, 1))
    n = G.gconv_bwd_weight_workspace(d)
    assert n > 0 and n % (16 * 9 * 4) == 0 and n // (16 * 9 * 4) <= 512
    # one thread per weight element (fp32): weights that alone fill the chip need no partial sums
    big = G.make_desc(2, "f32", 64, 8, 1024, 1024, (14, 14), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_bwd_weight_workspace(big) == 0
    # the matrix-core route (bf16, 128-channel groups): a few chunks of partial sums per weight
    tiled = G.make_desc(2, "bf16", 64, 8, 1024, 1024, (14, 14), (3, 3), (1, 1), (1, 1), (1, 1))
    wbytes = 1024 * 9 * 128 * 4
    n = G.gconv_bwd_weight_workspace(tiled)
    assert n % wbytes == 0 and 2 <= n // wbytes <= 64
    bad = G.make_desc(2, "f16", 1, 3, 8, 9, (9, 9), (3, 3), (1, 1), (1, 1), (1, 1))   # C % G != 0
    with pytest.raises(G.GconvError):
        G.gconv_bwd_weight_workspace(bad)
    assert G.gconv_bwd_weight(bad, 16, 16, 16, None, 0) == G.GCONV_ERR_BAD_DESC
    assert G.gconv_bwd_weight(d, 0, 16, 16, None, 0) == G.GCONV_ERR_NULL_PTR
    assert G.gconv_bwd_weight(d, 16, 17, 16, None, 0) == G.GCONV_ERR_MISALIGNED


def test_large_batch_splits_into_whole_image_launches():
    # a batch of x with >= 2^31 elements is valid; selection and plans describe one launch
    d = G.make_desc(2, "f16", 33, 64, 64, 64, (1024, 1024), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_validate(d) == G.GCONV_OK
    assert G.gconv_select_path(d) == G.GCONV_PATH_DEPTHWISE
    plan = G.gconv_get_plan(d)
    small = G.make_desc(2, "f16", 31, 64, 64, 64, (1024, 1024), (3, 3), (1, 1), (1, 1), (1, 1))
    assert plan == G.gconv_get_plan(small)        # (2^31 - 1) // 2^27 bytes = 15 images per launch
    fifteen = G.make_desc(2, "f16", 15, 64, 64, 64, (1024, 1024), (3, 3), (1, 1), (1, 1), (1, 1))
    assert plan == G.gconv_get_plan(fifteen)
    # backward weight reduces over the whole batch: a split batch needs a
    # chunk of partial sums per launch in the workspace
    assert G.gconv_bwd_weight(d, 16, 16, 16, None, 0) == G.GCONV_ERR_TOO_LARGE
    need = G.gconv_bwd_weight_workspace(d)
    assert need >= 3 * 64 * 9 * 4     # three launches (15 + 15 + 3 images), depthwise weights
    assert G.gconv_bwd_weight(d, 16, 16, 16, 32, 64 * 9 * 4 * 2) == G.GCONV_ERR_TOO_LARGE


# ---- the header as a plain C / C++ consumer sees it ------------------------

def _compiler(name):
    import shutil
    c = shutil.which(name)
    if c is None:
        pytest.skip("%s not available" % name)
    return c


@pytest.mark.parametrize("cc,flags,ext", [
    ("gcc", ["-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic"], ".c"),
    ("g++", ["-std=c++17", "-Wall", "-Wextra", "-Werror"], ".cpp"),
])
def test_header_compiles_alone(tmp_path, cc, flags, ext):
    import subprocess
    src = tmp_path / ("only_header" + ext)
    src.write_text('#include "gconv.h"\nint gconv_probe_unused(void) { return GCONV_ABI_VERSION; }\n')
    r = subprocess.run([_compiler(cc)] + flags + ["-I", os.path.dirname(HEADER), "-c", str(src),
                        "-o", str(tmp_path / "o.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_links_and_calls_host_functions(tmp_path):
    """A C99 caller linked against libgconv.so validates, sizes and routes
    every workload descriptor; the answers match the Python binding's."""
    import subprocess
    cc = _compiler("gcc")
    names = sorted(inputs.WORKLOADS)
    rows = []
    for n in names:
        d = G.desc_from_problem(inputs.WORKLOADS[n].problem)
        rows.append("{%d, %d, %d, %d, %d, %d, {%s}, {%s}, {%s}, {%s}, {%s}}" % (
            d.ndim, d.dtype, d.N, d.G, d.C, d.K,
            ", ".join(str(v) for v in d.in_), ", ".join(str(v) for v in d.filt),
            ", ".join(str(v) for v in d.stride), ", ".join(str(v) for v in d.pad),
            ", ".join(str(v) for v in d.dil)))
    prog = r'''
#include <stdio.h>
#include "gconv.h"
static const gconv_desc descs[] = { %s };
int main(void)
{
    unsigned i;
    if (gconv_abi_version() != GCONV_ABI_VERSION) return 3;
    for (i = 0; i < sizeof descs / sizeof descs[0]; ++i) {
        int64_t out[3];
        size_t ws = 0;
        int v = gconv_validate(&descs[i]);
        int o = gconv_out_dims(&descs[i], out);
        int p = gconv_select_path(&descs[i]);
        int b = gconv_bwd_weight_workspace(&descs[i], &ws);
        if (v != GCONV_OK || o != GCONV_OK || p < 0 || b != GCONV_OK) return 4;
        printf("%%d %%lld %%lld %%lld %%s %%lu\n", v, (long long)out[0], (long long)out[1],
               (long long)out[2], gconv_path_name(p), (unsigned long)ws);
    }
    printf("%%s\n", gconv_status_str(GCONV_ERR_BAD_DESC));
    return 0;
}
''' % ",\n    ".join(rows)
    src = tmp_path / "caller.c"
    src.write_text(prog)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(G.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src),
                        "-L", libdir, "-lgconv", "-Wl,-rpath," + libdir, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr)
    lines = r.stdout.strip().splitlines()
    assert len(lines) == len(names) + 1
    for n, line in zip(names, lines):
        d = G.desc_from_problem(inputs.WORKLOADS[n].problem)
        v, o0, o1, o2, path, ws = line.split()
        assert int(v) == G.GCONV_OK
        assert (int(o0), int(o1), int(o2)) == G.gconv_out_dims(d)
        assert path == G.gconv_path_name(G.gconv_select_path(d)) == EXPECTED_PATH[n]
        assert int(ws) == G.gconv_bwd_weight_workspace(d)
    assert lines[-1] == G.gconv_status_str(G.GCONV_ERR_BAD_DESC)


def test_half_batch_between_2_30_and_2_31_elements_stays_on_the_mfma_path():
    # x of 6000 large-group bf16 images: 1.2e9 elements (2.4 GB), over the
    # 2^31-byte reach of one launch's buffer offsets, so the batch is split
    # into launches that the halo implicit GEMM still takes
    d = G.make_desc(2, "bf16", 6000, 8, 1024, 1024, (14, 14), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_validate(d) == G.GCONV_OK
    assert G.gconv_path_name(G.gconv_select_path(d)) == "ighalo_mfma"
    one = G.make_desc(2, "bf16", 64, 8, 1024, 1024, (14, 14), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_select_path(one) == G.gconv_select_path(d)


def test_image_beyond_one_launch_is_split_into_slices():
    # one fp16 depthwise image of 6000 x 6000 x 64 = 2.3 G elements (4.6 GB):
    # launches of output row slices, each on the vector path it would take
    big = G.make_desc(2, "f16", 1, 64, 64, 64, (6000, 6000), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_validate(big) == G.GCONV_OK
    assert G.gconv_path_name(G.gconv_select_path(big)) == "depthwise"
    assert G.gconv_path_supported(big, G.GCONV_PATH_DEPTHWISE) == 1
    # the same in 3D splits along the planes
    big3 = G.make_desc(3, "bf16", 1, 8, 64, 64, (600, 240, 240), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert G.gconv_validate(big3) == G.GCONV_OK
    assert G.gconv_select_path(big3) >= 0
    # backward data accepts it as well (dx slices with the dy slices reaching them)
    assert G.gconv_bwd_data_workspace(big) == 64 * 9 * 2
    # backward weight runs the forward call's launches (three row slices of
    # up to 2794 rows here), each adding its own chunks of partial sums: the
    # workspace holds the same number of chunks for each, and fewer chunks
    # than launches is refused before any launch
    chunk = 64 * 9 * 4
    need = G.gconv_bwd_weight_workspace(big)
    assert need > 0 and need % (3 * chunk) == 0
    assert G.gconv_bwd_weight(big, 16, 16, 16, None, 0) == G.GCONV_ERR_TOO_LARGE
    assert G.gconv_bwd_weight(big, 16, 16, 16, 32, 2 * chunk) == G.GCONV_ERR_TOO_LARGE
    big3w = G.make_desc(3, "bf16", 1, 8, 16, 16, (600, 480, 480), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    need3 = G.gconv_bwd_weight_workspace(big3w)
    assert need3 > 0 and need3 % (3 * 16 * 27 * 2 * 4) == 0


def test_noalloc_entry_validates_before_any_hip_call():
    # a batch split into 5 launches needs 5 x 9.4 MB of partial sums > the 32 MiB scratch
    d = G.make_desc(2, "bf16", 40, 1, 512, 512, (512, 512), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_bwd_weight_noalloc(d, 256, 256, 256) == G.GCONV_ERR_SCRATCH
    assert "scratch" in G.gconv_status_str(G.GCONV_ERR_SCRATCH)
    assert G.gconv_bwd_weight_noalloc(d, 0, 256, 256) == G.GCONV_ERR_NULL_PTR
    bad = G.make_desc(2, "f16", 1, 3, 8, 9, (9, 9), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_bwd_weight_noalloc(bad, 256, 256, 256) == G.GCONV_ERR_BAD_DESC


def test_fp32_grouped_problems_leave_the_generic_kernel():
    # fp32 small groups whose 16-channel output tiles form 16-byte chunks
    # (ResNeXt-shaped 8/8, 3-channel groups are not): the LDS ring with fp32
    # MFMAs, in 2D and 3D
    d = G.make_desc(2, "f32", 32, 32, 256, 256, (56, 56), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "smallg_mfma"
    d = G.make_desc(3, "f32", 8, 32, 64, 128, (8, 28, 28), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "smallg_mfma"
    # groups of 4k channels: the implicit GEMM with fp32 MFMAs; 32-channel
    # tiles when 128-channel ones would leave fewer than 128 workgroups
    d = G.make_desc(2, "f32", 32, 8, 1024, 1024, (56, 56), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma"
    d = G.make_desc(3, "f32", 1, 1, 256, 256, (4, 28, 28), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma"
    assert G.gconv_get_plan(d)["grid"][1] == 8
    # odd group widths: the VALU direct kernel; on it, the wave-uniform-weight
    # variant for wide groups over many workgroups
    d = G.make_desc(2, "f32", 32, 32, 96, 96, (56, 56), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "direct_valu"
    assert G.gconv_tile_count(d, G.GCONV_PATH_DIRECT)[1] == 0
    d = G.make_desc(2, "f32", 32, 8, 1024, 1024, (56, 56), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_tile_count(d, G.GCONV_PATH_DIRECT)[1] == 4
    # too little work to fill the chip: the generic kernel's split reductions
    d = G.desc_from_problem(inputs.WORKLOADS["grouped2d_small_f32"].problem)
    assert G.gconv_path_name(G.gconv_select_path(d)) == "generic"
    assert G.gconv_path_supported(d, G.GCONV_PATH_DIRECT) == 1


def test_tile_menus():
    # depthwise: run lengths 4, 7, 14, 28 (stride 1) / 4, 7, 14 (stride 2)
    n, pk = G.gconv_tile_count(G.desc_from_problem(inputs.WORKLOADS["depthwise2d_f16"].problem))
    assert n == 4 and 0 <= pk < 4
    n, pk = G.gconv_tile_count(G.desc_from_problem(inputs.WORKLOADS["depthwise2d_s2_f16"].problem))
    assert n == 3 and 0 <= pk < 3
    # small groups 2D stride 1: ring with 14 or 28 rows, then the other variants that apply
    d = G.desc_from_problem(inputs.WORKLOADS["grouped2d_resnext_bf16"].problem)
    n, pk = G.gconv_tile_count(d)
    assert n >= 3 and pk in (0, 1)
    # generic: 1, 2, 4, 8, 16 threads per output, on any problem
    assert G.gconv_tile_count(d, G.GCONV_PATH_GENERIC)[0] == 5
    # a path that cannot take the problem, and AUTO on the tile entry, are errors
    with pytest.raises(G.GconvError):
        G.gconv_tile_count(d, G.GCONV_PATH_DEPTHWISE)
    assert G.gconv_fwd_tile(d, G.GCONV_PATH_AUTO, 0, 256, 256, None, 512) == G.GCONV_ERR_BAD_PATH
    assert G.gconv_fwd_tile(d, G.GCONV_PATH_SMALLG, n, 256, 256, None, 512) == G.GCONV_ERR_BAD_PATH
    # the plan of the own pick does not depend on a tile choice made before
    assert G.gconv_get_plan(d) == G.gconv_get_plan(d, G.gconv_select_path(d))


def test_half_type_groups_off_the_32_channel_grid_take_the_implicit_gemm():
    # widths of 8k input / 4k output channels that neither the small-group nor
    # the halo kernels take run the M-tiled implicit GEMM (K walked in chunks)
    for nd, Cpg, Kpg, G_ in ((3, 16, 32, 32), (2, 24, 24, 16), (2, 40, 48, 4), (2, 56, 56, 8),
                             (2, 16, 12, 7), (2, 8, 32, 16)):
        sp, fl = ((8, 14, 14), (3, 3, 3)) if nd == 3 else ((28, 28), (3, 3))
        one = (1,) * nd
        d = G.make_desc(nd, "bf16", 4, G_, G_ * Cpg, G_ * Kpg, sp, fl, one, one, one)
        assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma", (nd, Cpg, Kpg)
        n, pk = G.gconv_tile_count(d, G.GCONV_PATH_IGEMM)
        assert n >= 2 and 0 <= pk < n
    # channel counts off the 8-channel grid stay off the matrix cores
    d = G.make_desc(2, "bf16", 4, 8, 8 * 12, 8 * 32, (28, 28), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_path_supported(d, G.GCONV_PATH_IGEMM) == 0
    # the large-group workloads keep their 32-channel tile menu (BN x KT dividing Kpg x Cpg)
    d = G.desc_from_problem(inputs.WORKLOADS["grouped2d_large_bf16"].problem)
    assert G.gconv_tile_count(d, G.GCONV_PATH_IGEMM)[0] == 6


def test_generic_kernel_splits_long_reductions_of_small_outputs():
    # 200k outputs of 1728-long reductions: 8 threads per output (the 4th tile)
    d = G.make_desc(3, "f32", 1, 8, 512, 512, (4, 28, 28), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1))
    assert G.gconv_tile_count(d, G.GCONV_PATH_GENERIC) == (5, 3)
    # the fp32 implicit GEMM takes it (92 against 128 us in the fp32 sweep)
    assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma"


def test_dilated_small_groups_without_a_row_variant_take_the_implicit_gemm():
    # 8-channel groups, 3x3 dilation 2: only the small-group halo box would
    # take it, and the chunked implicit GEMM measured faster
    d = G.make_desc(2, "bf16", 11, 32, 256, 256, (28, 28), (3, 3), (1, 1), (2, 2), (2, 2))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma"
    assert G.gconv_path_supported(d, G.GCONV_PATH_SMALLG) == 1
    # the same without dilation streams rows on the small-group kernel
    d = G.make_desc(2, "bf16", 11, 32, 256, 256, (28, 28), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "smallg_mfma"


def test_selection_rules_from_the_held_out_sweep():
    # fp32 large groups with few pixels: on the VALU direct path, the
    # register-blocked kernel on 4-channel blocks (8-channel blocks would
    # leave too few threads); the menu is the per-thread kernel with
    # 8/4/2/1-channel blocks, then the wave-uniform-weight kernel with the
    # same blocks.  The dispatcher sends it to the fp32 implicit GEMM.
    d = G.make_desc(3, "f32", 1, 1, 256, 256, (4, 28, 28), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert G.gconv_tile_count(d, G.GCONV_PATH_DIRECT) == (8, 1)
    assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma"
    # depthwise on 7-row images: runs of 7 rows (none past the image, none ragged)
    d = G.make_desc(2, "bf16", 256, 384, 384, 384, (7, 7), (3, 3), (1, 1), (1, 1), (1, 1))
    assert G.gconv_tile_count(d, G.GCONV_PATH_DEPTHWISE)[1] == 1
    d = G.make_desc(2, "f32", 164, 96, 96, 96, (14, 14), (3, 3), (2, 2), (1, 1), (1, 1))
    assert G.gconv_tile_count(d, G.GCONV_PATH_DEPTHWISE)[1] == 1
    # a 7x7 image under a dilation-2 window is mostly halo: M-tiled GEMM
    d = G.make_desc(2, "f16", 235, 2, 512, 512, (7, 7), (3, 3), (1, 1), (2, 2), (2, 2))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "igemm_mfma"
    # the dilation-2 large-group workload keeps the halo kernel (18x18 box for 14x14)
    d = G.desc_from_problem(inputs.WORKLOADS["grouped2d_large_dil2_bf16"].problem)
    assert G.gconv_path_name(G.gconv_select_path(d)) == "ighalo_mfma"


def test_ring_tiles_of_four_chunks_and_3d_run_lengths():
    # half-type groups of 32 input channels per 16-channel output tile
    # (4-in/2-out; the 3D workload's backward-data problem) stream on the
    # ring; the menu is 7-row runs, 2-row runs, then the halo box
    d = G.make_desc(3, "f16", 8, 32, 128, 64, (8, 28, 28), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert G.gconv_path_name(G.gconv_select_path(d)) == "smallg_mfma"
    assert G.gconv_tile_count(d, G.GCONV_PATH_SMALLG) == (3, 0)
    assert G.gconv_get_plan(d)["grid"][0] == 512
    # the 3D workload: 7-row runs at N=8 (512 workgroups); at N=1 those
    # would leave fewer workgroups than CUs, so 2-row runs (224)
    d8 = G.desc_from_problem(inputs.WORKLOADS["grouped3d_f16_n8"].problem)
    assert G.gconv_tile_count(d8, G.GCONV_PATH_SMALLG) == (3, 0)
    assert G.gconv_get_plan(d8)["grid"][0] == 512
    d1 = G.desc_from_problem(inputs.WORKLOADS["grouped3d_f16_n1"].problem)
    assert G.gconv_tile_count(d1, G.GCONV_PATH_SMALLG) == (3, 1)
    assert G.gconv_get_plan(d1)["grid"][0] == 224


def test_bwd_weight_chunks_fill_one_round():
    # ResNeXt-style: 4 tiles of 4-wave workgroups per chunk, 128 chunks =
    # 512 workgroups, one round at two per CU; the workspace holds 128
    # chunks of fp32 partial sums of the 32 x 8 x 9 x 8 weights
    d = G.desc_from_problem(inputs.WORKLOADS["grouped2d_resnext_bf16"].problem)
    assert G.gconv_bwd_weight_workspace(d) == 128 * (32 * 8 * 9 * 8) * 4
