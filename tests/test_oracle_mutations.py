"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of the C oracle's source
(on the CPU, in a temporary directory), builds it, and checks that the
brute-force comparison, the hand example or the transpose invariant rejects it.
The oracle shipped in oracle/ is not touched.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import brute
import ss2d_inputs

SRC = os.path.join(os.path.dirname(oracle.__file__), "ss2d_oracle.c")

MUTATIONS = {
    "drop_skip_term": ("out[l] = Ds[c] * u[l];", "out[l] = 0.0;"),
    "wrong_sign_of_A": ("const double A = -exp(", "const double A = -1.0 + 0.0 * exp("),
    "column_walk_as_row_walk": ("return row * W + col;", "return col * H + row;"),
    "reverse_not_reversed": ("(k >= 2) ? (L - 1 - l) : l", "l"),
    "softplus_is_exp": ("return log1p(exp(v));", "return exp(v);"),
    "output_before_update": ("h = exp(delta[l] * A) * h + delta[l] * Bp[l] * u[l];\n          out[l] += Cp[l] * h;",
                             "out[l] += Cp[l] * h;\n          h = exp(delta[l] * A) * h + delta[l] * Bp[l] * u[l];"),
    "channel_index_swapped": ("const int64_t c = (int64_t)k * D + d;", "const int64_t c = d * 4 + k;"),
    "B_and_C_swapped": ("delta[l] * Bp[l] * u[l];", "delta[l] * Cp[l] * u[l];"),
    "bias_dropped": ("softplus_f64(dtp[l] + dt_bias[c])", "softplus_f64(dtp[l])"),
}


def _pins_pass(lib) -> bool:
    # brute force on a non-square map, random A_log, several channels and states
    inp = ss2d_inputs.tiny_random(2, 2, 3, 4, 3, seed=5)
    inp["Ds"] = np.random.default_rng(1).standard_normal(inp["Ds"].shape)
    y = oracle.ss2d_f64(**inp, lib=lib)
    if not np.allclose(y, brute.ss2d(**inp), rtol=1e-10, atol=1e-12):
        return False
    # the hand example
    x = np.array([1.0, 2.0]).reshape(1, 1, 1, 2)
    y = oracle.ss2d_f64(x, np.zeros((1, 4, 1, 2)), np.zeros((4, 1)), np.full(4, math.log(math.e - 1)),
                        np.ones((1, 4, 1, 2)), np.ones((1, 4, 1, 2)), np.ones(4), lib=lib)
    e = math.e
    return bool(np.allclose(y.reshape(-1), [8 + 4 / e, 16 + 2 / e], rtol=1e-14))


def test_shipped_oracle_passes_the_pins():
    assert _pins_pass(oracle._load())


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} not found"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so),
                           str(mutant), "-lm"])
    lib = oracle.load_library(str(so))
    with np.errstate(all="ignore"):
        assert not _pins_pass(lib)
