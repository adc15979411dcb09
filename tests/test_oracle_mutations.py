"""Planted mistakes in a temporary copy of the oracle must be caught by the pins.

Each mutation is applied to a copy of oracle/kda_oracle.c in a temp directory, compiled
with gcc and swapped in for the duration of the check; the real oracle is never touched.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_bwd_pins as bwd_pins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

DECAY_BLOCK = """  /* 1. per-channel decay of the old memory */
  for (int c = 0; c < K; ++c) {
    const double a = exp(g[c]);
    double* row = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) row[j] *= a;
  }
"""
READ_BLOCK_HEAD = "  /* 4. read with the query after the write */\n"

MUTATIONS = {
    "no_decay": [("row[j] *= a;", "row[j] *= 1.0;")],
    "gate_sign": [("const double a = exp(g[c]);", "const double a = exp(-g[c]);")],
    "no_beta": [("const double bk = beta * k[c];", "const double bk = k[c];")],
    "no_erase": [("row[j] += bk * (v[j] - u[j]);", "row[j] += bk * (v[j]);")],
    "erase_sign": [("row[j] += bk * (v[j] - u[j]);", "row[j] += bk * (v[j] + u[j]);")],
    "transposed_read": [("for (int j = 0; j < V; ++j) o[j] += row[j] * qc;",
                         "for (int j = 0; j < V; ++j) o[c < V ? c : 0] += row[j] * q[j < K ? j : 0] * (c < V);")],
    "decay_after_write": [(DECAY_BLOCK, ""), (READ_BLOCK_HEAD, DECAY_BLOCK + READ_BLOCK_HEAD)],
    "transposed_key_in_prediction": [("u[j] += row[j] * kc;", "u[j] += row[j] * k[j < K ? j : 0] * (c == 0);")],
    # planted in the gradients
    "bwd_du_sign": [("dS1[(size_t)c * V + j] = Lam[(size_t)c * V + j] - kt[c] * dr[j];",
                     "dS1[(size_t)c * V + j] = Lam[(size_t)c * V + j] + kt[c] * dr[j];")],
    "bwd_no_decay_on_adjoint": [("Lam[(size_t)c * V + j] = a * dS1[(size_t)c * V + j];",
                                 "Lam[(size_t)c * V + j] = dS1[(size_t)c * V + j];")],
    "bwd_dlog_alpha_without_alpha": [("dg[th * K + c] = a * acc;", "dg[th * K + c] = acc;")],
    "bwd_dq_from_previous_state": [("acc += Scur[(size_t)c * V + j] * dot[j];",
                                    "acc += Sprev[(size_t)c * V + j] * dot[j];")],
    "bwd_output_grad_added_after_use": [
        ("      for (int c = 0; c < K; ++c)\n        for (int j = 0; j < V; ++j) Lam[(size_t)c * V + j] += qt[c] * dot[j];\n", ""),
        ("      /* dlog a and L_{t-1} = Diag(a) dS' */\n",
         "      for (int c = 0; c < K; ++c)\n        for (int j = 0; j < V; ++j) dS1[(size_t)c * V + j] += qt[c] * dot[j];\n      /* dlog a and L_{t-1} = Diag(a) dS' */\n")],
    "bwd_missing_prediction_term_in_dk": [("        dk[th * K + c] += acc;\n", "")],
}

BWD_PIN_TESTS = [
    lambda: bwd_pins.test_gradients_match_central_differences([7], 2, 3, 4),
    lambda: bwd_pins.test_gradients_match_central_differences([4, 0, 6], 1, 4, 3),
    lambda: bwd_pins.test_zero_beta_closed_forms(),
]

PIN_TESTS = [
    lambda: pins.test_hand_example(),
    lambda: pins.test_bruteforce_dplr(3, 5, 7),
    lambda: pins.test_beta_zero_is_pure_decay(),
    lambda: pins.test_unit_key_beta_one_recalls_value(),
    lambda: pins.test_alpha_one_orthonormal_keys_is_linear_attention(),
    lambda: pins.test_basis_keys_are_per_channel_gated_attention(),
    lambda: pins.test_first_order_in_beta_is_diagonal_decay_attention(),
    lambda: pins.test_scalar_gate_is_gated_delta_rule(),
]


def _build_mutant(edits, tmp):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, "mutation anchor not found: %r" % old[:60]
        src = src.replace(old, new, 1)
    c = os.path.join(tmp, "m.c")
    so = os.path.join(tmp, "m.so")
    open(c, "w").write(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", so, c, "-lm"],
                   check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    oracle._load()
    real = oracle._lib
    tmp = tempfile.mkdtemp()
    try:
        lib = ctypes.CDLL(_build_mutant(MUTATIONS[name], tmp))
        for fn in ("kda_oracle_fwd", "kda_oracle_step", "kda_oracle_bwd"):
            getattr(lib, fn).argtypes = getattr(real, fn).argtypes
            getattr(lib, fn).restype = ctypes.c_int
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        oracle._lib = lib
        caught = []
        for i, t in enumerate(BWD_PIN_TESTS if name.startswith("bwd_") else PIN_TESTS):
            try:
                t()
            except AssertionError:
                caught.append(i)
        assert caught, "mutation %s survived every pin" % name
    finally:
        oracle._lib = real
        shutil.rmtree(tmp, ignore_errors=True)


def test_unmutated_copy_passes_every_pin():
    """Control: the same harness with no edit passes all pins."""
    oracle._load()
    real = oracle._lib
    tmp = tempfile.mkdtemp()
    try:
        lib = ctypes.CDLL(_build_mutant([], tmp))
        for fn in ("kda_oracle_fwd", "kda_oracle_step", "kda_oracle_bwd"):
            getattr(lib, fn).argtypes = getattr(real, fn).argtypes
            getattr(lib, fn).restype = ctypes.c_int
        oracle._lib = lib
        for t in PIN_TESTS + BWD_PIN_TESTS:
            t()
    finally:
        oracle._lib = real
        shutil.rmtree(tmp, ignore_errors=True)


# ---------------------------------------------------------------- the input prologue (numpy)
OPTION_PINS = [
    lambda: pins.test_log_sigmoid_values(),
    lambda: pins.test_sigmoid_values(),
    lambda: pins.test_l2_normalize_values(),
    lambda: pins.test_scalar_gate_option_is_gated_delta_rule(),
    lambda: pins.test_gate_logits_with_tiny_beta_is_pure_decay(),
    lambda: pins.test_l2norm_and_saturated_beta_recall_values(),
    lambda: pins.test_l2norm_option_is_scale_invariant_and_matches_numpy_norm(),
]

_real_apply = oracle.apply_options


def _apply_ignoring(bit):
    return lambda q, k, g, b, options: _real_apply(q, k, g, b, options & ~bit)


PROLOGUE_MUTATIONS = {
    "log_sigmoid_sign": ("log_sigmoid", lambda z: np.logaddexp(0.0, -np.asarray(z, dtype=np.float64))),
    "log_sigmoid_of_minus_z": ("log_sigmoid", lambda z: -np.logaddexp(0.0, np.asarray(z, dtype=np.float64))),
    "sigmoid_of_minus_x": ("sigmoid", lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, dtype=np.float64)))),
    "l2_without_sqrt": ("l2_normalize", lambda x, eps=1e-6: np.asarray(x) / (np.sum(np.asarray(x) ** 2, axis=-1, keepdims=True) + eps)),
    "l2_over_wrong_axis": ("l2_normalize", lambda x, eps=1e-6: np.asarray(x) / np.sqrt(np.sum(np.asarray(x) ** 2, axis=0, keepdims=True) + eps)),
    "gate_logits_ignored": ("apply_options", _apply_ignoring(oracle.OPT_GATE_LOGITS)),
    "beta_logits_ignored": ("apply_options", _apply_ignoring(oracle.OPT_BETA_LOGITS)),
    "l2norm_ignored": ("apply_options", _apply_ignoring(oracle.OPT_L2NORM_QK)),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTATIONS))
def test_option_pins_catch_prologue_mutation(name, monkeypatch):
    attr, fn = PROLOGUE_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for i, t in enumerate(OPTION_PINS):
        try:
            t()
        except (AssertionError, ValueError):
            caught.append(i)
    assert caught, "mutation %s survived every option pin" % name
