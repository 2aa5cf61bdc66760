"""The pins are sharp: copies of the oracle with one planted mistake each must fail
at least one pin. The mistakes are planted by text substitution in a temporary copy of
``oracle/kda_oracle.c`` compiled on the CPU; the committed oracle is never modified."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

DECAY = """        /* decay: row d of the state is scaled by 2^g[d] */
        for (int d = 0; d < K; ++d) {
            const double a = exp2(gt[d]);
            for (int c = 0; c < V; ++c)
                S[(size_t)d * V + c] *= a;
        }
"""
PREDICT = """        /* prediction p = S^T k */
        for (int c = 0; c < V; ++c)
            p[c] = 0.0;
        for (int d = 0; d < K; ++d)
            for (int c = 0; c < V; ++c)
                p[c] += kt[d] * S[(size_t)d * V + c];
"""
CORRECT = """        /* correction delta = beta (v - p) */
        for (int c = 0; c < V; ++c)
            delta[c] = bt * (vt[c] - p[c]);
"""
UPDATE = """        /* rank-one update S += k delta^T */
        for (int d = 0; d < K; ++d)
            for (int c = 0; c < V; ++c)
                S[(size_t)d * V + c] += kt[d] * delta[c];
"""
READ = """        /* read-out from the updated state: o = scale S^T q */
        for (int c = 0; c < V; ++c) {
            double acc = 0.0;
            for (int d = 0; d < K; ++d)
                acc += qt[d] * S[(size_t)d * V + c];
            ot[c] = J->scale * acc;
        }
"""

MUTANTS = {
    "gate_on_value_axis": ("const double a = exp2(gt[d]);\n            for (int c = 0; c < V; ++c)\n                S[(size_t)d * V + c] *= a;",
                           "for (int c = 0; c < V; ++c)\n                S[(size_t)d * V + c] *= exp2(gt[c % K]);"),
    "natural_exp": ("const double a = exp2(gt[d]);", "const double a = exp(gt[d]);"),
    "beta_outside": ("delta[c] = bt * (vt[c] - p[c]);", "delta[c] = bt * vt[c] - p[c];"),
    "no_beta": ("delta[c] = bt * (vt[c] - p[c]);", "delta[c] = (vt[c] - p[c]);"),
    "update_sign": ("S[(size_t)d * V + c] += kt[d] * delta[c];", "S[(size_t)d * V + c] -= kt[d] * delta[c];"),
    "read_with_key": ("acc += qt[d] * S[(size_t)d * V + c];", "acc += kt[d] * S[(size_t)d * V + c];"),
    "predict_with_query": ("p[c] += kt[d] * S[(size_t)d * V + c];", "p[c] += qt[d] * S[(size_t)d * V + c];"),
    "gva_modulo": ("const int h = hv / (HV / H);", "const int h = hv % H;"),
    "missing_scale": ("ot[c] = J->scale * acc;", "ot[c] = acc;"),
    "ignore_initial_state": ("memcpy(S, h0s, sizeof(double) * (size_t)K * V);", "memset(S, 0, sizeof(double) * (size_t)K * V);"),
    "packed_off_by_one": ("bos = J->cu[n];", "bos = J->cu[n] + (J->cu[n] < J->cu[n + 1]);"),
    "dense_batch_rows": ("row0 = (long)n * T;", "row0 = 0;"),
    "v_by_qk_head": ("const double *vt = J->v + (r * HV + hv) * V;", "const double *vt = J->v + (r * HV + h) * V;"),
    "beta_by_qk_head": ("const double bt = J->beta[r * HV + hv];", "const double bt = J->beta[r * HV + h];"),
    "no_decay": (
        "        /* decay: row d of the state is scaled by 2^g[d] */\n        for (int d = 0; d < K; ++d) {",
        "        for (int d = 0; d < K; ++d) {\n            break;"),
    "read_before_write": (UPDATE + READ, READ + UPDATE),
    "decay_after_update": (DECAY + PREDICT + CORRECT + UPDATE, PREDICT + CORRECT + UPDATE + DECAY),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", str(c),
                    "-o", str(so), "-lm"], check=True)
    return oracle.load_library(str(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)

    def impl(q, k, v, g, beta, h0, cu, scale):
        return oracle.recurrent(q, k, v, g, beta, h0, cu, scale, nthreads=1, lib=lib)

    failed = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    lib = _build_mutant(tmp_path, "identity", "#include <math.h>", "#include <math.h>")

    def impl(q, k, v, g, beta, h0, cu, scale):
        return oracle.recurrent(q, k, v, g, beta, h0, cu, scale, nthreads=1, lib=lib)

    for pin in pins.ALL_PINS:
        pin(impl)
