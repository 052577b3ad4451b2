"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source
(never in the GPU path), builds it, and re-runs the pin suite against it; the
suite has to fail.  Mistakes covered: step order, eps placement, clamp, every
term of the reverse step, the normalisation backward, the gate chain, the GQA
mapping, the checkpoint index, the masked-step semantics, the per-channel gate
(row vs column, its gradient's factor and state, the carry, masking, head
index), and in the conv
update of the decode path: tap order, window position, state carry, SiLU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTATIONS = {
    "read_before_decay": (
        "      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->gt.g;\n"
        "    for (int64_t c = 0; c < Dv; ++c) {\n      double acc = 0.0;\n"
        "      for (int64_t i = 0; i < Dk; ++i) acc += S[i * Dv + c] * s->khat[i];",
        "      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= 1.0;\n"
        "    for (int64_t c = 0; c < Dv; ++c) {\n      double acc = 0.0;\n"
        "      for (int64_t i = 0; i < Dk; ++i) acc += S[i * Dv + c] * s->khat[i];\n"
        "      for (int64_t i = 0; i < Dk; ++i) S[i * Dv + c] *= s->gt.g;"),
    "eps_outside_root": ("1.0 / sqrt(ss + ORACLE_EPS)", "1.0 / (sqrt(ss) + ORACLE_EPS)"),
    "eps_times_width": ("1.0 / sqrt(ss + ORACLE_EPS)", "1.0 / sqrt(ss + n * ORACLE_EPS)"),
    "no_clamp": ("r.xc = r.x < ORACLE_CLAMP ? r.x : ORACLE_CLAMP;", "r.xc = r.x;"),
    "dg_uses_decayed_state": ("dg += dSp[e] * Sprev[e];", "dg += dSp[e] * Sp[e];"),
    "dk_drops_state_term": (
        "acc += D[i * Dv + cc] * w.delta[cc] + Sp[i * Dv + cc] * du[cc];",
        "acc += D[i * Dv + cc] * w.delta[cc];"),
    "norm_bwd_no_projection": ("out[i] = r * (acc[i] - xhat[i] * dotp);", "out[i] = r * acc[i];"),
    "da_no_sigmoid": ("da[gi] = dl * (-s.gt.lam) * sigmoid(s.gt.xc) * pass;",
                      "da[gi] = dl * (-s.gt.lam) * pass;"),
    "dA_log_sign": ("dAl_part[gi] = dl == 0.0 ? 0.0 : dl * s.gt.ell;",
                    "dAl_part[gi] = dl == 0.0 ? 0.0 : -dl * s.gt.ell;"),
    "carry_without_decay": ("for (size_t e = 0; e < SS; ++e) D[e] = g * dSp[e];",
                            "for (size_t e = 0; e < SS; ++e) D[e] = dSp[e];"),
    "dbeta_uses_v": ("dbeta += ddel[cc] * (vt[cc] - w.u[cc]);", "dbeta += ddel[cc] * vt[cc];"),
    "q_not_scaled": ("s->qt[i] = scale * s->qhat[i];", "s->qt[i] = s->qhat[i];"),
    "dq_from_previous_state": ("acc += St[i * Dv + cc] * dOt[cc];",
                               "acc += Sprev[i * Dv + cc] * dOt[cc];"),
    "masked_step_decays": (
        "  if (s->valid) {\n    for (int64_t i = 0; i < Dk; ++i)\n"
        "      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->gt.g;",
        "  for (int64_t i = 0; i < Dk; ++i)\n"
        "      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->gt.g;\n"
        "  if (s->valid) {\n    if (0) {}"),
    "gqa_modulo": ("int64_t G = d->Hv / d->Hk, j = h / G;",
                   "int64_t G = d->Hv / d->Hk, j = h % d->Hk; (void)G;"),
    "ckpt_index": ("if (ckpt && (t + 1) % ORACLE_CKPT == 0 && t + 1 < d->T) {",
                   "if (ckpt && t % ORACLE_CKPT == 0 && t > 0 && t + 1 < d->T) {"),
    "beta_sign": ("r.beta = sigmoid(b);", "r.beta = sigmoid(-b);"),
    "db_chain": ("db[gi] = dbeta * beta * (1.0 - beta);", "db[gi] = dbeta * beta;"),
    "group_sum_first_head_only": ("for (int64_t hh = j * G; hh < (j + 1) * G; ++hh) {",
                                  "for (int64_t hh = j * G; hh < j * G + 1; ++hh) {"),
    "vg_gate_on_columns": ("for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->g[i];",
                           "for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->g[c % Dk];"),
    "vg_recompute_gate_on_columns": ("Sp[i * Dv + cc] = s.g[i] * Sprev[i * Dv + cc];",
                                     "Sp[i * Dv + cc] = s.g[cc % Dk] * Sprev[i * Dv + cc];"),
    "vg_dlg_no_gate_factor": ("dlt[i] = s.g[i] * acc;", "dlt[i] = acc;"),
    "vg_dlg_uses_decayed_state": (
        "for (int64_t cc = 0; cc < Dv; ++cc) acc += dSp[i * Dv + cc] * Sprev[i * Dv + cc];",
        "for (int64_t cc = 0; cc < Dv; ++cc) acc += dSp[i * Dv + cc] * Sp[i * Dv + cc];"),
    "vg_carry_without_decay": (
        "for (int64_t cc = 0; cc < Dv; ++cc) D[i * Dv + cc] = s.g[i] * dSp[i * Dv + cc];",
        "for (int64_t cc = 0; cc < Dv; ++cc) D[i * Dv + cc] = dSp[i * Dv + cc];"),
    "vg_masked_step_decays": (
        "  if (s->valid) {\n    for (int64_t i = 0; i < Dk; ++i)\n"
        "      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->g[i];",
        "  for (int64_t i = 0; i < Dk; ++i)\n"
        "      for (int64_t c = 0; c < Dv; ++c) S[i * Dv + c] *= s->g[i];\n"
        "  if (s->valid) {\n    if (0) {}"),
    "vg_gate_head_index": ("return ((size_t)(b * d->T + t) * d->Hv + h) * d->Dk;",
                           "return ((size_t)(b * d->T + t) * d->Hv + h / (d->Hv / d->Hk)) * d->Dk;"),
    "conv_taps_reversed": ("z += w[c * K + j] * ext[s + 1 + j];",
                           "z += w[c * K + (K - 1 - j)] * ext[s + 1 + j];"),
    "conv_window_one_late": ("z += w[c * K + j] * ext[s + 1 + j];", "z += w[c * K + j] * ext[s + j];"),
    "conv_state_not_advanced": ("final_state[row * K + j] = ext[S + j];", "final_state[row * K + j] = ext[j];"),
    "conv_no_silu": ("out[row * S + s] = z * sigmoid(z);", "out[row * S + s] = z;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert old in src, "mutation pattern no longer matches the oracle source"
    c = tmp_path / "m.c"
    so = tmp_path / "m.so"
    c.write_text(src.replace(old, new, 1))
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(c), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode != 0, "pins did not catch mutation %s" % name
