"""Planted mistakes in a copy of the oracle must each fail at least one pin (CPU only).

Every mutant is a plausible slip in the oracle's arithmetic -- a dropped term, a
wrong sign, a transposed operand, a wrong index -- applied to a temporary copy
of ``oracle/mlstm_oracle.c`` and compiled with gcc.  The real oracle is never
modified.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS, BWD_PINS, EPI_PINS, SLSTM_PINS

MUTANTS = {
    "forget_gate_dropped_on_C": (
        "row[j] = f_s * row[j] + i_s * v[r] * k[j];",
        "row[j] = row[j] + i_s * v[r] * k[j];"),
    "outer_product_transposed": (
        "row[j] = f_s * row[j] + i_s * v[r] * k[j];",
        "row[j] = f_s * row[j] + i_s * v[j % dv] * k[r % dqk];"),
    "stabilizer_sign": (
        "const double f_s = exp(log_f + m_prev - m_t);",
        "const double f_s = exp(log_f - m_prev - m_t);"),
    "stabilizer_max_dropped": (
        "const double m_t = fmax(log_f + m_prev, log_i);",
        "const double m_t = log_f + m_prev;"),
    "input_gate_not_exponential": (
        "const double i_s = exp(log_i - m_t);",
        "const double i_s = (log_i - m_t);"),
    "forget_gate_not_log": (
        "const double log_f = log_sigmoid(f_pre);",
        "const double log_f = sigmoid(f_pre);"),
    "naive_log_sigmoid": (
        "return fmin(x, 0.0) - log1p(exp(-fabs(x)));",
        "return log(1.0 / (1.0 + exp(-x)));"),
    "normalizer_abs_dropped": (
        "fmax(fabs(nq), exp(-m_t))",
        "fmax(nq, exp(-m_t))"),
    "normalizer_floor_sign": (
        "fmax(fabs(nq), exp(-m_t))",
        "fmax(fabs(nq), exp(m_t))"),
    "normalizer_floor_unstabilized": (
        "fmax(fabs(nq), exp(-m_t))",
        "fmax(fabs(nq), 1.0)"),
    "normalizer_no_decay": (
        "n[j] = f_s * n[j] + i_s * k[j];",
        "n[j] = n[j] + i_s * k[j];"),
    "retrieval_with_key": (
        "cq += row[j] * q[j];",
        "cq += row[j] * k[j];"),
    "output_gate_dropped": (
        "h[r] = sigmoid(o_pre[r]) * cq / denom;",
        "h[r] = cq / denom;"),
    "head_stride": (
        "double *Cb = C + (size_t)bh * dv * dqk;",
        "double *Cb = C + (size_t)bh * dqk;"),
    # backward
    "bwd_normalizer_sign": (
        "dden[t] = fabs(den[t]) > 1.0 ? -(den[t] > 0 ? 1.0 : -1.0) * dun / (N * N) : 0.0;",
        "dden[t] = fabs(den[t]) > 1.0 ? (den[t] > 0 ? 1.0 : -1.0) * dun / (N * N) : 0.0;"),
    "bwd_floor_ignored": (
        "dden[t] = fabs(den[t]) > 1.0 ? -(den[t] > 0 ? 1.0 : -1.0) * dun / (N * N) : 0.0;",
        "dden[t] = -(den[t] > 0 ? 1.0 : -1.0) * dun / (N * N);"),
    "bwd_output_gate_derivative": (
        "doh[e] = dhh[e] * u * g * (1.0 - g);",
        "doh[e] = dhh[e] * u * g;"),
    "bwd_value_grad_without_score": (
        "dvh[(size_t)s * dv + r] += d * sc * dnum[(size_t)t * dv + r];",
        "dvh[(size_t)s * dv + r] += d * dnum[(size_t)t * dv + r];"),
    "bwd_key_side_decay_dropped": (
        "                dF[s] -= dl;\n",
        ""),
    "bwd_forget_cumsum_forward": (
        "for (int j = S - 1; j >= 0; --j) {",
        "for (int j = 0; j < S; ++j) {"),
    "bwd_log_sigmoid_derivative": (
        "dfh[j] = rev * sigmoid(-fh[j]);",
        "dfh[j] = rev * sigmoid(fh[j]);"),
    # block epilogue
    "epi_unbiased_variance": (
        "var /= dv;",
        "var /= (dv - 1);"),
    "epi_shift_dropped": (
        "* inv + gn_b[c] + skip_w[c]",
        "* inv + skip_w[c]"),
    "epi_skip_ungated": (
        "(gn_w[c] * (hr[r] - mu) * inv + gn_b[c] + skip_w[c] * x[row + r]) * g;",
        "(gn_w[c] * (hr[r] - mu) * inv + gn_b[c]) * g + skip_w[c] * x[row + r];"),
    "epi_mean_not_subtracted": (
        "gn_w[c] * (hr[r] - mu) * inv",
        "gn_w[c] * hr[r] * inv"),
    "epi_channel_ignores_head": (
        "const size_t c = (size_t)hd * dv + r;",
        "const size_t c = r;"),
    "epi_swish_as_sigmoid": (
        ": z[row + r] * sigmoid(z[row + r]);",
        ": sigmoid(z[row + r]);"),
    # sLSTM
    "slstm_recurrent_transposed": (
        "for (int j = 0; j < dh; ++j) acc += row[j] * hp[j];",
        "for (int j = 0; j < dh; ++j) acc += Rh[((size_t)g * dh + j) * dh + r] * hp[j];"),
    "slstm_gate_order": (
        "ai = a[dh + r], af = a[2 * dh + r]",
        "ai = a[2 * dh + r], af = a[dh + r]"),
    "slstm_cell_input_not_squashed": (
        "c[r] = fs * c[r] + is * tanh(az);",
        "c[r] = fs * c[r] + is * az;"),
    "slstm_normalizer_no_forget": (
        "n[r] = fs * n[r] + is;",
        "n[r] = n[r] + is;"),
    "slstm_head_ignored": (
        "const int hd = bh % NH;",
        "const int hd = 0;"),
    "slstm_stabilizer_max_dropped": (
        "const double m_t = fmax(log_f + m[r], ai);",
        "const double m_t = log_f + m[r];"),
    "slstm_output_gate_dropped": (
        "ht[r] = sigmoid(ao) * c[r] / n[r];",
        "ht[r] = c[r] / n[r];"),
    "slstm_hidden_not_fed_back": (
        "            for (int r = 0; r < dh; ++r) hp[r] = ht[r];\n",
        ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(str(mutated), lib_path)
    orc = oracle.Oracle(oracle.load(lib_path))
    failed = []
    for pin in ALL_PINS + BWD_PINS + EPI_PINS + SLSTM_PINS:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
