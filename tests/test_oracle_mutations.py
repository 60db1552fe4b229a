"""Plant a plausible mistake in a copy of oracle.c and require the pins to
catch it.  Each mutation is a dropped term, a wrong sign or index, a transposed
operand or a misplaced constant; the unmodified oracle passes every pin
(test_oracle.py), so a pin failure here is caused by the planted mistake."""
import os
import tempfile

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "dropped_softmax_scale": ("logits[j] = scale * dot;", "logits[j] = dot;"),
    "causal_mask_leaks_next_row": (
        "const int64_t n_keys = pos[i] + 1;",
        "const int64_t n_keys = (pos[i] + 2 < kv_rows) ? pos[i] + 2 : kv_rows;"),
    "gqa_modulo_mapping": ("const int g = h / group;", "const int g = h % hkv;"),
    "eps_outside_root": ("sqrt(sum_sq / (double)d + eps)", "(sqrt(sum_sq / (double)d) + eps)"),
    "rms_sum_not_mean": ("sqrt(sum_sq / (double)d + eps)", "sqrt(sum_sq + eps)"),
    "rms_divides_by_d_minus_1": ("sqrt(sum_sq / (double)d + eps)",
                                 "sqrt(sum_sq / (double)(d - 1) + eps)"),
    "gain_dropped": ("* g / rms;", "/ rms;"),
    "weight_transposed": ("read_elem(w, w_dtype, c * ncols + j)", "read_elem(w, w_dtype, j * d + c)"),
    "no_max_subtraction": ("logits[j] = exp(logits[j] - m);", "logits[j] = exp(logits[j]);"),
    "missing_normalisation": ("o[q_base + e] = acc[e] / l;", "o[q_base + e] = acc[e];"),
    "lse_without_max": ("lse[i * hq + h] = m + log(l);", "lse[i * hq + h] = log(l);"),
    "v_reads_k": ("acc[e] += logits[j] * read_elem(v, kv_dtype, v_base + e);",
                  "acc[e] += logits[j] * read_elem(k, kv_dtype, v_base + e);"),
    "dot_skips_last_element": ("for (int e = 0; e < dh; ++e) {\n          dot +=",
                               "for (int e = 0; e < dh - 1; ++e) {\n          dot +="),
    "rope_sin_sign": ("xh[j0] = a * c - b * s;", "xh[j0] = a * c + b * s;"),
    "rope_frequency_exponent": ("pow(theta, -2.0 * (double)i / (double)dh)", "pow(theta, -1.0 * (double)i / (double)dh)"),
    "rope_position_off_by_one": ("(double)pos[r] * freq", "(double)(pos[r] + 1) * freq"),
    "rope_pairing_swapped": ("const int j0 = interleaved ? 2 * i : i;", "const int j0 = interleaved ? i : 2 * i;"),
    "bwd_softmax_jacobian_term_dropped": ("const double ds = (exp(x[j] - m) / l) * (dp[j] - d_term);",
                                          "const double ds = (exp(x[j] - m) / l) * dp[j];"),
    "bwd_dk_missing_scale": ("dk[kv_base + e] += scale * ds * read_elem(q, q_dtype, q_base + e);",
                             "dk[kv_base + e] += ds * read_elem(q, q_dtype, q_base + e);"),
    "bwd_dv_unnormalised": ("const double p = exp(scale * qk - stat_m[t]) / stat_l[t];",
                            "const double p = exp(scale * qk - stat_m[t]);"),
    "bwd_causal_boundary_exclusive": ("const int64_t j_end = pos[i] + 1 < j1 ? pos[i] + 1 : j1;",
                                      "const int64_t j_end = pos[i] < j1 ? pos[i] : j1;"),
    "bwd_gqa_modulo_mapping": ("for (int h = g * group; h < (g + 1) * group; ++h) {",
                               "for (int h = g; h < hq; h += hkv) {"),
    "bwd_dq_reads_v": ("dq[q_base + e] += ds * read_elem(k, kv_dtype, kv_base + e);",
                       "dq[q_base + e] += ds * read_elem(v, kv_dtype, kv_base + e);"),
    "bwd_rms_projection_term_dropped": ("dx[r * d + c] = g * dy[r * d + c] / rr[r] - xv / ((double)d * r3) * proj;",
                                        "dx[r * d + c] = g * dy[r * d + c] / rr[r];"),
    "bwd_rms_cubed_as_squared": ("const double r3 = rr[r] * rr[r] * rr[r];", "const double r3 = rr[r] * rr[r];"),
    "bwd_dgain_missing_rms": ("ag += dy[r * d + c] * read_elem(x, x_dtype, r * d + c) / rr[r];",
                              "ag += dy[r * d + c] * read_elem(x, x_dtype, r * d + c);"),
    "bwd_dw_uses_unnormalised_x": ("ak += y[r * d + c] * read_elem(dz_k, dz_dtype, r * ncols + j);",
                                   "ak += read_elem(x, x_dtype, r * d + c) * read_elem(dz_k, dz_dtype, r * ncols + j);"),
    "gret_decay_applied_before_use": (
        "        for (int e = 0; e < dv; ++e) out[e] += decay * dot * read_elem(v, dtype, (m * heads + h) * dv + e);\n        decay *= gamma[m * heads + h];",
        "        decay *= gamma[m * heads + h];\n        for (int e = 0; e < dv; ++e) out[e] += decay * dot * read_elem(v, dtype, (m * heads + h) * dv + e);"),
    "gret_gate_exponent_inverted": ("gamma[i] = pow(sig, 1.0 / tau);", "gamma[i] = pow(sig, tau);"),
    "gret_start_state_not_decayed": ("out[e] += decay * acc;", "out[e] += acc;"),
    "gret_step_reads_old_state": (
        "s[c * dv + e] = gm * s[c * dv + e] + kc * read_elem(v, dtype, bh * dv + e);",
        "s[c * dv + e] = s[c * dv + e];"),
    "gret_state_outer_product_transposed": (
        "for (int e = 0; e < dv; ++e) s[c * dv + e] += kc * read_elem(v, dtype, (m * heads + h) * dv + e);",
        "for (int e = 0; e < dv; ++e) s[c * dv + e] += kc * read_elem(v, dtype, (m * heads + h) * dv + c % dv);"),
    "gret_final_state_skips_first_token": ("for (int64_t m = n - 1; m >= 0; --m) {", "for (int64_t m = n - 1; m >= 1; --m) {"),
    "bwd_dy_weight_transposed": ("read_elem(w_k, w_dtype, c * ncols + j);", "read_elem(w_k, w_dtype, j * d + c);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"oracle_{name}.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(force=True, src=path, out=os.path.join(tmp, f"lib_{name}.so"))
        mutant = oracle.Oracle(lib)
        caught = []
        for pin in ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, MemoryError) as exc:
                caught.append((pin.__name__, str(exc)[:80]))
        assert caught, f"no pin caught the planted mistake {name}"
