"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/gconv_ref.c`` (flipped
filter, dropped bias, wrong group in the input index, transposed weight
operand, stride and dilation swapped, wrong sign of the padding, a dropped
absolute value in the error scale, an off-by-one output extent), builds it
with gcc into a temporary directory and checks that the brute-force scatter
pin or the extent pin of ``test_oracle_pins`` rejects it.  CPU only.
"""
import os
import shutil

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import brute_extent, scatter_conv, small_int_problem

SRC = os.path.join(os.path.dirname(oracle.__file__), "gconv_ref.c")

MUTANTS = {
    "flipped_filter": ("+ xx * dil[2];", "+ (X - 1 - xx) * dil[2];"),
    "dropped_bias": ("acc += b;", "acc += 0.0 * b;"),
    "wrong_input_group": ("* W + iw) * G + g) * Cpg + c;", "* W + iw) * G + (g + 1) % G) * Cpg + c;"),
    "transposed_weight": ("int64_t wi = ((((g * Kpg + k) * Z + z) * Y + yy) * X + xx) * Cpg + c;",
                          "int64_t wi = ((((g * Cpg + c) * Z + z) * Y + yy) * X + xx) * Kpg + k;"),
    "stride_dil_swapped": ("oh * stride[1] - pad[1] + yy * dil[1]", "oh * dil[1] - pad[1] + yy * stride[1]"),
    "pad_sign": ("ow * stride[2] - pad[2]", "ow * stride[2] + pad[2]"),
    "scale_without_abs": ("s += fabs(t);", "s += t;"),
    "extent_off_by_one": ("return room / stride + 1;", "return (room + stride - 1) / stride + 1;"),
}


def _caught(lib) -> bool:
    for n, k, s, p, d in [(5, 3, 2, 1, 1), (8, 3, 3, 0, 1), (6, 2, 2, 1, 2), (7, 3, 2, 2, 1)]:
        if oracle.out_extent(n, k, s, p, d, lib) != brute_extent(n, k, s, p, d):
            return True
    for case in range(24):
        rng = np.random.default_rng(7000 + case)
        x, w, b, G, st, pd, dl = small_int_problem(rng, 2 if case % 2 else 3)
        try:
            y, sc = oracle.conv_fwd(x, w, b, G, st, pd, dl, lib=lib)
        except ValueError:
            return True
        y_ref, s_ref = scatter_conv(x, w, b, G, st, pd, dl)
        if y.shape != y_ref.shape or not np.array_equal(y, y_ref) or not np.array_equal(sc, s_ref):
            return True
    return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished from the oracle: %s" % name
    mutated = tmp_path / ("gconv_ref_%s.c" % name)
    mutated.write_text(src.replace(old, new, 1))
    lib = oracle.bind(oracle.build(src=str(mutated), out=str(tmp_path / ("lib_%s.so" % name))))
    assert _caught(lib), "pins did not catch mutant %s" % name


def test_unmutated_passes():
    assert not _caught(oracle._load())
