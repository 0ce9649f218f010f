"""Strength of the oracle's pins: copies of the oracle with one planted mistake
(built on the CPU into a temporary directory) must each fail at least one pin.

Each mutation is a plausible slip in one step: a dropped term, a wrong sign,
index or operand, a transposed weight, a missing rounding."""
import os
import subprocess

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTATIONS = {
    "conv_taps_reversed": ("pre += wc[m] * wn[m];", "pre += wc[W - 2 - m] * wn[m];"),
    "conv_bias_dropped": ("double pre = bias ? bias[c] : 0.0;", "double pre = 0.0;"),
    "conv_silu_dropped": ("y[c] = pre * kda_ref_sigmoid(pre);", "y[c] = pre;"),
    "conv_window_not_shifted": ("if (W > 1) wn[W - 2] = x[c];", ";"),
    "gate_dt_bias_dropped": ("(g1 + dt_bias[i])", "(g1)"),
    "gate_a_log_head_index": ("exp(A_log[i / KDA_REF_HEAD_DIM])", "exp(A_log[0])"),
    "gate_f_b_transposed": ("f_b[(int64_t)i * KDA_REF_FA_RANK + m]",
                            "f_b[(int64_t)m * KDA_REF_FA_RANK + i % KDA_REF_FA_RANK]"),
    "gate_no_exp_on_a_log": ("double a = exp(A_log[i / KDA_REF_HEAD_DIM]);",
                             "double a = A_log[i / KDA_REF_HEAD_DIM];"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "l2norm_eps_outside_sqrt": ("double inv = 1.0 / sqrt(ss + eps);",
                                "double inv = 1.0 / (sqrt(ss) + eps);"),
    "recur_decay_by_row": ("row[i] *= exp(g[i]);", "row[i] *= exp(g[j % dk]);"),
    "recur_u_sign": ("double bu = beta * (v[j] - kS);", "double bu = beta * (v[j] + kS);"),
    "recur_update_uses_q": ("row[i] += bu * k[i];", "row[i] += bu * q[i];"),
    "recur_beta_dropped": ("double bu = beta * (v[j] - kS);", "double bu = (v[j] - kS);"),
    "rmsnorm_sum_not_mean": ("double rstd = 1.0 / sqrt(ss / (double)n + eps);",
                             "double rstd = 1.0 / sqrt(ss + eps);"),
    "rmsnorm_gate_dropped": ("y[j] = o[j] * rstd * w[j] * kda_ref_sigmoid(gate[j]);",
                             "y[j] = o[j] * rstd * w[j];"),
    "verify_reads_first_slot": ("*src = row[a - 1];", "*src = row[0];"),
    "state_not_carried_rounded": ("Sh[e] = (double)f;", ";"),
    "conv_window_written_reversed": (
        "p->conv[dst[t] * p->conv_slot_stride + c * p->conv_dim_stride + m * p->conv_pos_stride] =",
        "p->conv[dst[t] * p->conv_slot_stride + c * p->conv_dim_stride + (W - 2 - m) * p->conv_pos_stride] ="),
    "beta_head_index": ("x[4 * (int64_t)D + KDA_REF_FA_RANK + h]", "x[4 * (int64_t)D + KDA_REF_FA_RANK]"),
    "q_scale_on_k": ("kda_ref_l2norm(N, y + D + (int64_t)h * N, p->l2_eps, 1.0, kh);",
                     "kda_ref_l2norm(N, y + D + (int64_t)h * N, p->l2_eps, p->q_scale, kh);"),
    "bf16_truncates": ("double r = nearbyint(a / q) * q;", "double r = floor(a / q) * q;"),
    "gate_reads_gate_columns": ("kda_ref_gate(H, fb, x + 4 * (int64_t)D,",
                                "kda_ref_gate(H, fb, x + 3 * (int64_t)D,"),
    "linear_drops_last_k": ("for (int32_t k = 0; k < K; ++k) acc += xr[k] * kda_ref_bf16_to_double(wr[k]);",
                            "for (int32_t k = 0; k + 1 < K; ++k) acc += xr[k] * kda_ref_bf16_to_double(wr[k]);"),
    "linear_weight_transposed": ("const uint16_t* wr = w + (int64_t)n * K;\n            double acc",
                                 "const uint16_t* wr = w + (int64_t)n;\n            double acc"),
    "linear_ignores_pitch": ("for (int32_t k = 0; k < K; ++k) xr[k] = kda_ref_bf16_to_double(x[(int64_t)m * x_pitch + k]);",
                             "for (int32_t k = 0; k < K; ++k) xr[k] = kda_ref_bf16_to_double(x[(int64_t)m * K + k]);"),
    "handoff_conv_not_rounded": (
        "y[c] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(y[c]));   /* hand-off */", ";"),
    "handoff_g1_not_rounded": (
        "if (round_g1) g1 = kda_ref_bf16_to_double(kda_ref_double_to_bf16(g1));   /* hand-off */", ";"),
    "handoff_o_not_rounded": (
        "o[j] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(o[j]));   /* hand-off */", ";"),
    "handoff_rounds_k_hat_not_conv_out": (
        "y[c] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(y[c]));   /* hand-off */",
        "if (c >= D && c < 2 * D) y[c] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(y[c]));"),
    "tie_conv_margin_drops_bias": ("double mg = b ? fabs(b[c]) : 0.0, pre", "double mg = 0.0, pre"),
    "tie_conv_margin_drops_slope": ("cmag[c] = fabs(slope) * mg +", "cmag[c] = mg +"),
    "tie_g1_certificate_always_exact": ("if (mag == 0.0 || mag <= ldexp(q, 24)) return 0.0;",
                                        "return 0.0;"),
    "tie_o_margin_drops_delta_term": ("omag[j] = aq + fabs(beta) * (fabs(v[j]) + ak) * kq;",
                                      "omag[j] = aq;"),
    "tie_y_counted_on_wrong_head": ("++tr[h * 4 + 3];", "++tr[0 * 4 + 3];"),
    "tie_replay_conv_not_rounded": (
        "if (near_tie(y[c], rel[0] * cmag[c])) ++tr[((c % D) / N) * 4 + 0];\n"
        "                y[c] = kda_ref_bf16_to_double(kda_ref_double_to_bf16(y[c]));",
        "if (near_tie(y[c], rel[0] * cmag[c])) ++tr[((c % D) / N) * 4 + 0];"),
    "duplicate_threshold_off_by_one": ("if (count[dst[t]] > 1) collide[r] = 1;",
                                       "if (count[dst[t]] > 2) collide[r] = 1;"),
    "duplicate_within_row_ignored": (
        "for (int32_t t = 0; t < L; ++t) ++count[dst[t]];",
        "for (int32_t t = 0; t < L; ++t) count[dst[t]] = count[dst[t]] < r + 1 ? r + 1 : count[dst[t]] + 1;"),
    "duplicate_collider_not_skipped": (
        "if (resolve_slots(p, r, &src, dst) != 0 || collide[r]) { ++skipped; continue; }\n\n"
        "        /* Read the carried",
        "if (resolve_slots(p, r, &src, dst) != 0) { ++skipped; continue; }\n\n"
        "        /* Read the carried"),
}


# The near-tie replay (checker instrumentation) repeats some of the definition's
# expressions; a mutation named tie_* is planted in the replay, any other in the
# definition (everything before the replay's section).
REPLAY_MARK = "/* Near ties of the hand-off mode"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    cut = src.index(REPLAY_MARK)
    end = src.index("/* Projections around the core")
    if name.startswith("tie_"):
        head, region, tail = src[:cut], src[cut:end], src[end:]
    elif name.startswith("linear_"):
        head, region, tail = src[:end], src[end:], ""
    else:
        head, region, tail = "", src[:cut], src[cut:]
    assert region.count(old) == 1, f"mutation anchor not unique in its region: {old!r}"
    mutated = tmp_path / "kda_oracle_mutant.c"
    mutated.write_text(head + region.replace(old, new) + tail)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(lib), str(mutated), "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    caught = []
    for check in PINS:
        try:
            check(orc)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"
