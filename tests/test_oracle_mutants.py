"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped gate, a wrong sign, a transposed
operand, a swapped order of decay and erase, ...) into a copy of the oracle's C
source, builds that copy in a temporary directory, and runs the forward and
VJP pins against it: at least one pin must fail.  The unaltered source must
pass the same battery.  Nothing here touches the GPU.
"""
import os

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn2_oracle.c")

READ_BLOCK = """    /* read-out after the update */
    if (o) {
        for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            const double* row = S + c * dv;
            for (int64_t j = 0; j < dv; ++j) o[j] += row[j] * q[c];
        }
    }
"""
DECAY_LOOP = "        for (int64_t j = 0; j < dv; ++j) row[j] *= a;\n"

MUTANTS = {
    "decay_on_value_axis": [(DECAY_LOOP,
                             "        for (int64_t j = 0; j < dv; ++j) row[j] *= exp(g[j % dk]);"
                             " (void)a;\n")],
    "decay_sign": [("double a = exp(g[c]);\n        double* row = S + c * dv;",
                    "double a = exp(-g[c]);\n        double* row = S + c * dv;")],
    "read_without_erase_gate": [("double bk = b[c] * k[c];", "double bk = k[c];")],
    "read_with_gate_only": [("double bk = b[c] * k[c];", "double bk = b[c];")],
    "write_gate_dropped": [("u[j] = w[j] * v[j] - r[j];", "u[j] = v[j] - r[j];")],
    "write_gate_on_residual": [("u[j] = w[j] * v[j] - r[j];", "u[j] = w[j] * (v[j] - r[j]);")],
    "residual_sign": [("u[j] = w[j] * v[j] - r[j];", "u[j] = w[j] * v[j] + r[j];")],
    "erase_gate_on_write_side": [("row[j] += k[c] * u[j];", "row[j] += b[c] * k[c] * u[j];")],
    "transposed_write": [("row[j] += k[c] * u[j];", "row[j] += k[j % dk] * u[c % dv];")],
    "erase_reads_undecayed_state": [
        (DECAY_LOOP, "        (void)row; (void)a;\n"),
        ("    /* gated residual, then write along k */\n",
         "    for (int64_t c = 0; c < dk; ++c) {\n"
         "        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= exp(g[c]);\n    }\n"
         "    /* gated residual, then write along k */\n")],
    "readout_before_update": [
        (READ_BLOCK, ""),
        ("    /* gated residual, then write along k */\n",
         READ_BLOCK + "    /* gated residual, then write along k */\n")],
    "initial_state_ignored": [("if (j->s0) memcpy(S, j->s0 + task * dk * dv",
                               "if (0) memcpy(S, j->s0 + task * dk * dv")],
    # backward
    "vjp_dlogalpha_sign": [("acc_dg += dsp * sp;", "acc_dg -= dsp * sp;")],
    "vjp_missing_erase_term": [("double dsp = G[c * dv + jj] - kh * du[jj];",
                                "double dsp = G[c * dv + jj];")],
    "vjp_db_wrong_factor": [("db[c] = acc_dkh * k[c];", "db[c] = acc_dkh * b[c];")],
    "vjp_state_grad_not_decayed": [("G[c * dv + jj] = a * dSp[c * dv + jj];",
                                    "G[c * dv + jj] = dSp[c * dv + jj];")],
    "vjp_dq_from_previous_state": [("acc += Scur[c * dv + jj] * dO[jj];",
                                    "acc += Sprev[c * dv + jj] * dO[jj];")],
    "vjp_dw_dv_swapped": [("dw[jj] = du[jj] * v[jj];", "dw[jj] = du[jj] * w[jj];")],
}


def small_fd_check():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 6, 1, 3, 4
    q, k, v, g, b, w, S0 = pins.rand_inputs(rng, B, T, H, dk, dv, g_lo=-0.4)
    do = rng.standard_normal((B, T, H, dv))
    dsT = rng.standard_normal((B, H, dk, dv))
    grads = oracle.vjp(q, k, v, g, b, w, do, S0, dsT)
    args = dict(q=q, k=k, v=v, g=g, b=b, w=w, S0=S0)
    names = dict(q="dq", k="dk", v="dv", g="dlog_alpha", b="db", w="dw", S0="ds0")
    h = 1e-6
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = pins._loss(**args, do=do, dsT=dsT)
            x[idx] = old - h
            lm = pins._loss(**args, do=do, dsT=dsT)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(grads[names[name]] - fd).max() < 1e-6 * max(1.0, np.abs(fd).max()), name


BATTERY = [
    pins.test_dense_transition_products,
    pins.test_exact_rational_worked_example,
    pins.test_reduces_to_kda_when_gates_equal_scalar,
    pins.test_exact_retrieval_along_unit_key,
    pins.test_closed_form_geometric_decay,
    pins.test_gated_linear_attention_parallel_form,
    small_fd_check,
]


def run_battery():
    failures = []
    for fn in BATTERY:
        try:
            fn()
        except (AssertionError, RuntimeError, ValueError) as e:  # noqa: PERF203
            failures.append((fn.__name__, type(e).__name__))
    return failures


def _build_variant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, (name, "edit anchor must occur exactly once", old)
        src = src.replace(old, new)
    path = tmp_path / ("oracle_%s.c" % name)
    path.write_text(src)
    return oracle.build(src=str(path), out=str(tmp_path / ("lib_%s.so" % name)))


def test_unaltered_source_passes_battery(tmp_path):
    lib = _build_variant(tmp_path, "unaltered", [])
    with oracle.use_build(lib):
        assert run_battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    lib = _build_variant(tmp_path, name, MUTANTS[name])
    with oracle.use_build(lib):
        failures = run_battery()
    assert failures, "planted mistake %r passed every pin" % name
