"""Each plausible slip in the oracle must make a pin fail.

The test copies the oracle's C source, plants one mistake by text
substitution (a dropped term, a wrong sign, a wrong index, a flipped
comparison), builds that copy into a temporary library and runs the pin suite
against it in a child process. A mutant that passes every pin would mean the
pins cannot see that kind of mistake. Runs on the CPU only.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "tie_break_high_index": ("if (best < 0 || l[e] > l[best]) best = e;",
                             "if (best < 0 || l[e] >= l[best]) best = e;"),
    "drop_b1": ("a[(size_t)r * h + n] = silu(s + b);", "a[(size_t)r * h + n] = silu(s);"),
    "drop_b2": ("y[(size_t)r * d + m] = s + b;", "y[(size_t)r * d + m] = s;"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "w2_transposed": ("w[n] = widen(w2e, wdt, (size_t)m * h + n);",
                      "w[n] = widen(w2e, wdt, (size_t)n * d + m);"),
    "always_renorm": ("renorm ? pj / sel : pj", "pj / sel"),
    "capacity_zero_unlimited": ("if (capacity >= 0 && kept > capacity)",
                                "if (capacity > 0 && kept > capacity)"),
    "aux_missing_E": ("*loss = (double)E * s;", "*loss = s;"),
    "residual_dropped": ("double s = residual ? widen(residual, rdt, (size_t)tok[i] * d + m) : 0.0;",
                         "double s = 0.0;"),
    "router_bias_dropped": ("if (gate_bias) s += (double)gate_bias[e];", ""),
    "bf16_shift": ("uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;",
                   "uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 15;"),
    "softmax_no_shift_in_num": ("p[e] = exp(l[e] - m) / z;", "p[e] = exp(l[e]) / z;"),
    "combine_gate_ignored": ("s += gate[(size_t)i * k + j] * y_slots", "s += y_slots"),
    "drop_keeps_last": ("if (rank < kept) {", "if (rank >= counts[e] - kept) {"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(lib),
                    str(mut), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


# Slips in the backward oracle (numpy source), caught by its own pins.
BWD_SRC = os.path.join(ROOT, "oracle", "backward.py")
BWD_MUTANTS = {
    "silu_grad_drops_z_term": ("return s * (1.0 + z * (1.0 - s))", "return s"),
    "silu_grad_sign": ("return s * (1.0 + z * (1.0 - s))", "return s * (1.0 - z * (1.0 - s))"),
    "softmax_grad_no_centering": ("return p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                                  "return p * dp"),
    "renorm_no_centering": ("(gate * (dgate - inner)).ravel()", "(gate * dgate).ravel()"),
    "no_renorm_skips_softmax": ("return softmax_grad(softmax(lg), dp)\n\n\ndef aux_grad",
                                "return dp\n\n\ndef aux_grad"),
    "aux_over_T_once": ("np.broadcast_to(daux * E * counts.astype(np.float64) / (float(T) * T), (T, E))",
                        "np.broadcast_to(daux * E * counts.astype(np.float64) / float(T), (T, E))"),
    "aux_missing_E": ("np.broadcast_to(daux * E * counts.astype(np.float64) / (float(T) * T), (T, E))",
                      "np.broadcast_to(daux * counts.astype(np.float64) / (float(T) * T), (T, E))"),
    "dw2_from_preactivation": ("dw2 = dy.T @ a", "dw2 = dy.T @ z"),
    "db1_before_silu_grad": ("db1 = dz.sum(axis=0)", "db1 = da.sum(axis=0)"),
    "dx_misses_router": ("# logits = x W_g^T + b_g\n    dw_gate = dl.T @ X\n"
                         "    dgate_bias = None if gate_bias is None else dl.sum(axis=0)\n    dx += dl @ Wg",
                         "# logits = x W_g^T + b_g\n    dw_gate = dl.T @ X\n"
                         "    dgate_bias = None if gate_bias is None else dl.sum(axis=0)\n    dx = dx"),
    "ec_dx_misses_router": ("dl = softmax_grad(p, dgate)\n    dw_gate = dl.T @ X\n"
                            "    dgate_bias = None if gate_bias is None else dl.sum(axis=0)\n"
                            "    dx += dl @ Wg",
                            "dl = softmax_grad(p, dgate)\n    dw_gate = dl.T @ X\n"
                            "    dgate_bias = None if gate_bias is None else dl.sum(axis=0)\n"
                            "    dx = dx"),
    "dgate_from_scaled_dy": ("dgate[slots] = (dO[tok] * y).sum(axis=1)",
                             "dgate[slots] = (dy * y).sum(axis=1)"),
    "residual_gradient_dropped": ("dx = dO.copy() if residual else np.zeros((T, d), np.float64)",
                                  "dx = 0.0 * dO if residual else np.zeros((T, d), np.float64)"),
    "ec_residual_gradient_dropped": ("dx = dO.copy() if residual else np.zeros((T, d))",
                                     "dx = 0.0 * dO if residual else np.zeros((T, d))"),
    "dy_ignores_gate": ("dy = gflat[slots][:, None] * dO[tok]", "dy = dO[tok]"),
    "dx_reversed_columns": ("dx = dz @ w1e", "dx = dz @ w1e[:, ::-1]"),
    "ec_no_softmax_backward": ("dl = softmax_grad(p, dgate)", "dl = dgate"),
    "ec_ungated_dy": ("dy = gate[tok, e][:, None] * dO[tok]", "dy = dO[tok]"),
    "ec_gate_from_score": ("gate = np.where(dest >= 0, p, 0.0)", "gate = np.where(dest >= 0, 1.0, 0.0)"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = open(BWD_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "backward_mut.py"
    mut.write_text(src.replace(old, new))
    env = dict(os.environ, MOE_ORACLE_BWD=str(mut), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_backward.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


# Slips in the error yardsticks that set the GPU bounds (the magnitudes of
# backward.py), caught by the per-element
# definitions of tests/test_oracle_scales.py. An inflated yardstick would
# widen a GPU bound without failing any gradient or output pin.
SCALE_MUTANTS = {
    "scale_dw1_inflated": ('        m["dw1"][e] = adz.T @ aX[tok]',
                           '        m["dw1"][e] = 16.0 * (adz.T @ aX[tok])'),
    "scale_gate_dropped": ("        ady = np.abs(gflat[slots])[:, None] * aO[tok]",
                           "        ady = aO[tok]"),
    "scale_z_term_dropped": ('        adz = (ady @ np.abs(W2[e])) * (np.abs(silu_grad(z)) + np.abs(z) / 8.0)\n'
                             '        m["dw1"][e]',
                             '        adz = (ady @ np.abs(W2[e])) * np.abs(silu_grad(z))\n'
                             '        m["dw1"][e]'),
    "scale_router_centring_sign": ("(ag * (m_dg + inner)).ravel()", "(ag * (m_dg - inner)).ravel()"),
    "scale_aux_dropped": ("        m_dl = m_dl + p * (dpa + (p * dpa).sum(axis=1, keepdims=True))",
                          "        m_dl = m_dl"),
    "ec_scale_dw1_inflated": ('            mag["dw1"][e] = adz.T @ np.abs(X[tok])',
                              '            mag["dw1"][e] = 16.0 * (adz.T @ np.abs(X[tok]))'),
    "ec_scale_gate_dropped": ("            ady = np.abs(dy)", "            ady = np.abs(dO[tok])"),
    "ec_scale_softmax_dropped": ('        mdl = p * (mag["dgate"] + (p * mag["dgate"]).sum(axis=1, keepdims=True))',
                                 '        mdl = mag["dgate"]'),
}


def _run_scale_pins(env):
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_scales.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(SCALE_MUTANTS))
def test_scale_mutant_is_caught(name, tmp_path):
    old, new = SCALE_MUTANTS[name]
    src = open(BWD_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "backward_mut.py"
    mut.write_text(src.replace(old, new))
    r = _run_scale_pins(dict(os.environ, MOE_ORACLE_BWD=str(mut), OMP_NUM_THREADS="2"))
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
