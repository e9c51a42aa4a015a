"""The oracle's pins reject plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source, such as a
dropped term, a flipped sign, a wrong operand or index, or a missing decay
factor. It builds that copy with the same gcc line as the oracle and runs the
pins of ``test_oracle`` against it. At least one pin must fail. A control case
builds the unchanged source the same way and must pass every pin, so a failure
comes from the planted mistake and not from the harness.

The planted mistakes cover every stage of what the oracle computes:
- the forward recurrence (delta-rule write, decay, read-out, scale), from the
  FlashQLA GDN overview, sections 2 and 3;
- the adjoint recurrence;
- the L2-norm, sigmoid and gate backward, from the FlashKDA backward page,
  the prepare-backward section;
- the chunk checkpoints and the terminal state gradient;
- the grouped-head index, from the FlashQLA GDN overview, section 4.
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle as pins

_SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

# (name, gate the mistake is live under, exact source text, replacement)
MUTANTS = [
    ("write: v + e instead of v - e", 0,
     "(a->v[row * V + i] - e);\n      if (a->u_out)", "(a->v[row * V + i] + e);\n      if (a->u_out)"),
    ("forward: decay dropped", 0,
     "{ Si[j] *= dec[j]; e += Si[j] * knt[j]; }\n      const double u = beta[t] * (a->v[row * V + i] - e);\n"
     "      if (a->u_out)",
     "{ e += Si[j] * knt[j]; }\n      const double u = beta[t] * (a->v[row * V + i] - e);\n      if (a->u_out)"),
    ("read-out: k instead of q", 0, "o += Si[j] * qnt[j];", "o += Si[j] * knt[j];"),
    ("read-out: scale dropped", 0, "a->o[row * V + i] = a->scale * o;", "a->o[row * V + i] = o;"),
    ("dq: the u kn^T term dropped", 0,
     "dqt[j] += w * (Sti[j] + ut[i] * knt[j]);", "dqt[j] += w * Sti[j];"),
    ("de: sign flipped", 0, "const double de = -beta[t] * du[i];", "const double de = beta[t] * du[i];"),
    ("dk: the St^T de term dropped", 0,
     "{ dSi[j] += de * knt[j]; dkt[j] += Sti[j] * de; }", "{ dSi[j] += de * knt[j]; }"),
    ("dS: decay not carried back", 0,
     "{ dlt[j] += dSi[j] * Sti[j]; dSi[j] *= dec[j]; }", "{ dlt[j] += dSi[j] * Sti[j]; }"),
    ("dlam: k instead of the state", 0, "dlt[j] += dSi[j] * Sti[j];", "dlt[j] += dSi[j] * knt[j];"),
    ("L2 backward: projection dropped", 0,
     "rq[t] * (dqt[j] - qnt[j] * pq)", "rq[t] * dqt[j]"),
    ("L2 backward: q instead of k in the projection", 0,
     "pk += knt[j] * dkt[j];", "pk += qnt[j] * dkt[j];"),
    ("beta backward: sigmoid derivative missing a factor", 0,
     "dbeta[t] * beta[t] * (1.0 - beta[t])", "dbeta[t] * (1.0 - beta[t])"),
    ("softplus gate backward: sign flipped", 1,
     "dlt[j] * (-ea * sigmoid(x))", "dlt[j] * (ea * sigmoid(x))"),
    ("softplus gate: d A_log missing lambda", 1,
     "*pdA += dlt[j] * lam[(size_t)t * K + j];", "*pdA += dlt[j];"),
    ("sigmoid gate backward: derivative missing a factor", 2,
     "a->gate_scale * sz * (1.0 - sz)", "a->gate_scale * sz"),
    ("sigmoid gate: d A_log missing e^A_log", 2, "*pdA += dz * ea * x;", "*pdA += dz * x;"),
    ("recompute: every chunk starts from the first checkpoint", 0,
     "memcpy(S, ckpt + (size_t)c * VK, VK * sizeof(double));", "memcpy(S, ckpt, VK * sizeof(double));"),
    ("terminal state gradient dropped", 0,
     "if (a->dht) memcpy(dS, a->dht", "if (0) memcpy(dS, a->dht"),
    ("grouped heads: interleaved instead of consecutive", 0,
     "hk = h / (H / Hk);", "hk = h % Hk;"),
]


def _build(src_text: str, tmp_path, tag: str):
    c = tmp_path / f"{tag}.c"
    so = tmp_path / f"lib{tag}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-std=c99", "-O2", "-shared", "-fPIC", "-pthread", "-o", str(so), str(c), "-lm"],
                   check=True)
    lib = ctypes.CDLL(str(so))
    lib.oracle_run.argtypes = [ctypes.POINTER(oracle._Args)]
    lib.oracle_run.restype = ctypes.c_int
    return lib


def _battery(gate: int):
    """The pins that apply under ``gate``; returns the names of those that fail."""
    checks = [
        ("finite differences", lambda: pins.test_finite_differences_all_inputs(gate, [5, 11], 4)),
        ("literal matrix form", lambda: pins.test_forward_matches_literal_matrix_form(gate)),
        ("single-token closed form", lambda: pins.test_single_token_closed_form(gate)),
        ("beta = 0 reduction", lambda: pins.test_beta_zero_reduces_to_gated_linear_attention(gate)),
        ("L2 invariants", lambda: pins.test_l2_gradient_orthogonal_and_scale_invariant(gate)),
        ("grouped = repeated heads", lambda: pins.test_grouped_heads_equal_repeated_heads(gate)),
    ]
    failed = []
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_control_unchanged_source_passes(tmp_path, monkeypatch):
    src = open(_SRC).read()
    monkeypatch.setattr(oracle, "_lib", _build(src, tmp_path, "control"))
    for gate in (0, 1, 2):
        assert _battery(gate) == [], gate


@pytest.mark.parametrize("name,gate,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, gate, old, new, tmp_path, monkeypatch):
    src = open(_SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {name}"
    monkeypatch.setattr(oracle, "_lib", _build(src.replace(old, new), tmp_path, "mutant"))
    with np.errstate(all="ignore"):
        failed = _battery(gate)
    assert failed, f"no pin rejects: {name}"
