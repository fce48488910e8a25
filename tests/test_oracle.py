"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention)


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((4, 3)), np.zeros((5, 3)), np.zeros((4, 3)), False, 1.0)
    with pytest.raises(RuntimeError):
        oracle.attention(np.zeros((4, 3)), np.zeros((4, 3)), np.zeros((4, 3)), False, 1.0, rows=[4])


def test_oracle_reports_threads():
    assert oracle.num_threads() >= 1


# Plausible mistakes, planted into a copy of attention.c. Every one must fail a pin.
MUTANTS = {
    "causal_excludes_diagonal": ("if (causal && j > i)", "if (causal && j >= i)"),
    "causal_wrong_side": ("if (causal && j > i)", "if (causal && j < i)"),
    "scale_dropped": ("s_row[j] = scale * dot;", "s_row[j] = dot;"),
    "key_index_wrong": ("q[i * d + c] * k[j * d + c]", "q[i * d + c] * k[i * d + c]"),
    "scores_transposed": ("q[i * d + c] * k[j * d + c]", "q[j * d + c] * k[i * d + c]"),
    "normalisation_dropped": ("p_row[j] = exp(s_row[j] - m) / denom;", "p_row[j] = exp(s_row[j] - m);"),
    "max_missing_from_L": ("lse[r] = m + log(denom);", "lse[r] = log(denom);"),
    "denominator_unshifted": ("denom += exp(s_row[j] - m);", "denom += exp(s_row[j]);"),
    "value_index_wrong": ("acc += p_row[j] * v[j * d + c];", "acc += p_row[j] * v[i * d + c];"),
    "head_offset_dropped": ("const double *k = K + bh * N * d;", "const double *k = K;"),
    "row_list_ignored": ("const int64_t i = rows ? rows[r] : r;", "const int64_t i = r;"),
    "max_wrong_direction": ("if (s_row[j] > m) m = s_row[j];", "if (s_row[j] > m) m = s_row[0];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attention.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(mutant_c), "-lm"], check=True)
    lib = oracle.load_library(str(so))

    def attn(Q, K, V, causal, scale, rows=None):
        return oracle.attention(Q, K, V, causal, scale, rows=rows, lib=lib)

    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
