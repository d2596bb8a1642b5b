"""Plant plausible mistakes into copies of the oracle (on the CPU) and check
that every one of them trips at least one pin.  The real oracle source is
never modified: each mutant is a text edit of ``oracle/oracle.c`` compiled
into a temporary directory."""
import os

import pytest

import oracle
from oracle.oracle import _SRC, OracleLib
from pins import PINS

WRITE = "for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * u[j];"
READ_BLOCK = """    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
        o[j] = acc;
    }"""

# (name, [(old, new), ...]) — each `old` must occur in oracle.c exactly once.
MUTANTS = [
    ("delta_sign", [("u[j] = beta * (v[j] - vhat);", "u[j] = beta * (v[j] + vhat);")]),
    ("delta_no_beta", [("u[j] = beta * (v[j] - vhat);", "u[j] = (v[j] - vhat);")]),
    ("predict_with_query", [("vhat += k[i] * S[(size_t)i * dv + j];",
                             "vhat += q[i] * S[(size_t)i * dv + j];")]),
    ("read_with_key", [("acc += q[i] * S[(size_t)i * dv + j];",
                        "acc += k[i] * S[(size_t)i * dv + j];")]),
    ("read_before_write", [("    /* rank-one write k^T u */\n    for (i = 0; i < dk; ++i)\n        " + WRITE,
                            "    /* rank-one write moved below */"),
                           (READ_BLOCK, READ_BLOCK + "\n    for (i = 0; i < dk; ++i)\n        " + WRITE)]),
    ("gate_off_by_one", [("if (gate == ORACLE_GATE_SCALAR) gt = g + tok;",
                          "if (gate == ORACLE_GATE_SCALAR) gt = g + (t > 0 ? tok - 1 : tok);")]),
    ("beta_off_by_one", [("? beta[tok] : 0.0;", "? beta[t > 0 ? tok - 1 : tok] : 0.0;")]),
    ("channel_gate_reversed", [("double a = exp(g[i]);", "double a = exp(g[dk - 1 - i]);")]),
    ("channel_gate_first_only", [("double a = exp(g[i]);", "double a = exp(g[0]);")]),
    ("scalar_gate_not_exp", [("double a = exp(g[0]);", "double a = 1.0 + g[0];")]),
    ("ignore_initial_state", [("if (s0) memcpy(", "if (0) memcpy(")]),
    ("write_uses_v_not_u", [(WRITE, WRITE.replace("u[j]", "v[j]"))]),
    ("write_half", [(WRITE, WRITE.replace("k[i] * u[j]", "0.5 * k[i] * u[j]"))]),
    # Gated DeltaProduct
    ("gdp_substeps_reversed", [("for (j = 0; j < nh; ++j) {", "for (j = nh - 1; j >= 0; --j) {")]),
    ("gdp_decay_every_substep", [("                for (i = 0; i < dk * dv; ++i) S[i] *= a;\n            }\n"
                                  "            for (j = 0; j < nh; ++j) {",
                                  "            }\n            for (j = 0; j < nh; ++j) {\n"
                                  "                if (gate == ORACLE_GATE_SCALAR)\n"
                                  "                    for (i = 0; i < dk * dv; ++i) S[i] *= exp(g[tok]);")]),
    ("gdp_no_beta", [("w[c] = bj * (vj[c] - pred);", "w[c] = (vj[c] - pred);")]),
    ("gdp_first_key_only", [("const double *kj = k + (tok * nh + j) * dk;",
                             "const double *kj = k + (tok * nh) * dk;")]),
    ("gdp_beta_of_first_substep", [("double bj = beta[tok * nh + j];", "double bj = beta[tok * nh];")]),
    ("gdp_ignore_initial_state", [("if (s0 != NULL) memcpy(", "if (0) memcpy(")]),
    # normalised linear attention
    ("norm_no_decay_on_z", [("z[r] = a * z[r] + kt[r];", "z[r] = z[r] + kt[r];")]),
    ("norm_den_with_key", [("den += qt[r] * z[r];", "den += kt[r] * z[r];")]),
    ("norm_ignore_z0", [("if (z0 != NULL) memcpy(", "if (0) memcpy(")]),
    ("norm_ignore_s0", [("if (s0 != 0) memcpy(", "if (0) memcpy(")]),
    ("norm_channel_gate_reversed", [(": gate == ORACLE_GATE_CHANNEL ? exp(g[tok * dk + r]) : 1.0;",
                                     ": gate == ORACLE_GATE_CHANNEL ? exp(g[tok * dk + dk - 1 - r]) : 1.0;")]),
    ("norm_not_divided", [("o[tok * dv + c] = num / den;", "o[tok * dv + c] = num;")]),
    # backward pass
    ("bwd_dq_from_decayed_state", [("acc += dot[j] * St[(size_t)i * dv + j];",
                                    "acc += dot[j] * sd[(size_t)i * dv + j];")]),
    ("bwd_no_prediction_into_key", [("dk_out[tok * dk + i] += acc;", "dk_out[tok * dk + i] += 0.0 * acc;")]),
    ("bwd_prediction_sign", [("acc += sd[(size_t)i * dv + j] * (-bt * du[j]);",
                              "acc += sd[(size_t)i * dv + j] * (bt * du[j]);")]),
    ("bwd_no_correction_into_state", [("Hg[(size_t)i * dv + j] += kt[i] * (-bt * du[j]);",
                                       "Hg[(size_t)i * dv + j] += 0.0;")]),
    ("bwd_gate_not_passed_back", [("for (i = 0; i < dk * dv; ++i) Hg[i] *= a;", "(void)a;")]),
    ("bwd_dbeta_with_value_only", [("db += du[j] * (vt[j] - vh[j]);", "db += du[j] * vt[j];")]),
    ("bwd_dg_with_new_state", [("acc += Hg[i] * sd[i];", "acc += Hg[i] * St[i];")]),
    ("bwd_channel_dg_reversed", [("dg[tok * dk + i] = acc;", "dg[tok * dk + (dk - 1 - i)] = acc;")]),
    ("bwd_ignore_initial_state", [("if (s0 == NULL) memset(St,", "if (1) memset(St,")]),
    ("bwd_ignore_final_state_grad", [("if (dsT) memcpy(Hg,", "if (0) memcpy(Hg,")]),
    ("gdp_bwd_substeps_in_forward_order", [("for (j = nh - 1; j >= 0; --j) {", "for (j = 0; j < nh; ++j) {")]),
    ("gdp_bwd_dbeta_value_only", [("db += du[c] * (vj[c] - vh[c]);", "db += du[c] * vj[c];")]),
    ("gdp_bwd_no_prediction_into_state", [("Hg[(size_t)i * dv + c] -= kj[i] * bj * du[c];",
                                           "Hg[(size_t)i * dv + c] -= 0.0 * kj[i] * bj * du[c];")]),
    ("gdp_bwd_dg_with_token_end_state", [("for (i = 0; i < dk * dv; ++i) acc += Hg[i] * Sj[i];",
                                          "for (i = 0; i < dk * dv; ++i) acc += Hg[i] * St[i];")]),
    ("gdp_bwd_gate_not_passed_back", [("for (i = 0; i < dk * dv; ++i) Hg[i] = a * Hg[i];", "(void)a;")]),
    ("gdp_bwd_ignore_final_state_grad", [("if (dsT != NULL) memcpy(Hg,", "if (0) memcpy(Hg,")]),
    ("gdp_bwd_ignore_initial_state", [("if (NULL != s0) memcpy(St,", "if (0) memcpy(St,")]),
    ("gdp_bwd_dq_from_first_substep", [("acc += dot[c] * Sl[(size_t)i * dv + c];",
                                        "acc += dot[c] * Sj[(size_t)i * dv + c];")]),
    ("bwd_readout_grad_missing", [("Hg[(size_t)i * dv + j] += qt[i] * dot[j];", "Hg[(size_t)i * dv + j] += 0.0;")]),
]


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, edits):
    src = open(_SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
        src = src.replace(old, new)
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.build(force=True, src=path, out=os.path.join(tmp_path, f"lib{name}.so"))
    orc = OracleLib(lib)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
