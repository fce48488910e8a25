"""The cross-attention oracle against its pins (CPU only), and the pins against planted mistakes."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import pins_cross

# One plausible mistake per line of the definition: each must fail some pin.
MUTANTS = {
    "key_loop_uses_nq": ("for (int64_t j = 0; j < Nk; ++j) {\n        if (causal", "for (int64_t j = 0; j < Nq && j < Nk; ++j) {\n        if (causal"),
    "bottom_right_alignment": ("if (causal && j > i) {", "if (causal && j > i + Nk - Nq) {"),
    "causal_wrong_side": ("if (causal && j > i) {", "if (causal && j < i) {"),
    "scale_dropped": ("s_row[j] = scale * dot;", "s_row[j] = dot;"),
    "v_stride_uses_nq": ("const double *v = V + bh * Nk * d;", "const double *v = V + bh * Nq * d;"),
    "lse_without_max": ("lse[i] = m + log(denom);", "lse[i] = log(denom);"),
    "softmax_unnormalised": ("p_row[j] = exp(s_row[j] - m) / denom;", "p_row[j] = exp(s_row[j] - m);"),
}


def _attn(Q, K, V, causal, scale):
    return oracle.attention_cross(Q, K, V, causal, scale)


@pytest.mark.parametrize("pin", pins_cross.ALL_PINS, ids=lambda p: p.__name__)
def test_cross_oracle_pin(pin):
    pin(_attn)


def test_cross_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.attention_cross(np.zeros((1, 1, 3, 4)), np.zeros((1, 1, 5, 4)), np.zeros((1, 1, 4, 4)), False, 1.0)
    with pytest.raises(ValueError):
        oracle.attention_cross(np.zeros((1, 1, 3, 4)), np.zeros((1, 2, 5, 4)), np.zeros((1, 2, 5, 4)), False, 1.0)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_cross_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    here = os.path.dirname(oracle.__file__)
    src = open(os.path.join(here, "attention_cross.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    os.path.join(here, "attention.c"), str(mutant_c), "-lm"], check=True)
    lib = oracle.load_library(str(so))

    def attn(Q, K, V, causal, scale):
        return oracle.attention_cross(Q, K, V, causal, scale, lib=lib)

    caught = []
    for pin in pins_cross.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
