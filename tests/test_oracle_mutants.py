"""The oracle's pins catch plausible mistakes.

Each case rebuilds oracle.c on the CPU with one deliberate mistake (a wrong
sign, index, constant, rounding, dropped term or swapped operand) into a
temporary library and runs every pin against it in a child process.  The
case passes when at least one pin fails (or the child dies).  The oracle
source itself is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = [
    ("gamma_drops_abs", "sum += fabs((double)W[n * K + k]);", "sum += (double)W[n * K + k];"),
    ("gamma_wrong_count", "return (float)(sum / (double)(N * K));", "return (float)(sum / (double)(N * K + K));"),
    ("ternarize_multiplies", "float t = rintf(W[n * K + k] / d);", "float t = rintf(W[n * K + k] * d);"),
    ("ternarize_truncates", "float t = rintf(W[n * K + k] / d);", "float t = truncf(W[n * K + k] / d);"),
    ("ternarize_rounds_half_away", "float t = rintf(W[n * K + k] / d);", "float t = roundf(W[n * K + k] / d);"),
    ("pack_twos_complement", "uint8_t code = (uint8_t)(v + 1);", "uint8_t code = (uint8_t)(v & 3);"),
    ("pack_group_transposed", "int64_t grp = k / 16, j = k % 16, t = j % 4;", "int64_t grp = k / 16, j = k % 16, t = j / 4;"),
    ("rms_mean_off_by_one", "float ms = (float)(ss / (double)K);", "float ms = (float)(ss / (double)(K - 1));"),
    ("rms_eps_outside_root", "float r = 1.0f / sqrtf(ms + eps);", "float r = 1.0f / (sqrtf(ms) + eps);"),
    ("rms_drops_gain", "xn[k] = (orc_bf16_to_float(row[k]) * r) * g[k];", "xn[k] = (orc_bf16_to_float(row[k]) * r);"),
    ("quant_128", "float scale = 127.0f / (amax > 1e-5f ? amax : 1e-5f);", "float scale = 128.0f / (amax > 1e-5f ? amax : 1e-5f);"),
    ("quant_floor", "float v = rintf(xn[k] * scale);", "float v = floorf(xn[k] * scale);"),
    ("quant_absmax_signed", "float a = fabsf(xn[k]);", "float a = xn[k];"),
    ("accumulate_sign_swapped", "a -= q[m * K + k];", "a += q[m * K + k];"),
    ("accumulate_wrong_row", "if (w[n * K + k] == 1)", "if (w[((n + 1) % N) * K + k] == 1)"),
    ("rescale_inverted", "(double)acc[m * N + n] * (double)gamma / (double)s[m];", "(double)acc[m * N + n] * (double)s[m] / (double)gamma;"),
    ("rescale_wrong_token", "(double)gamma / (double)s[m];", "(double)gamma / (double)s[(m + 1) % M];"),
    ("glu_swaps_gate_up", "double gate = z[m * 2 * F + f];\n            double up = z[m * 2 * F + F + f];",
     "double up = z[m * 2 * F + f];\n            double gate = z[m * 2 * F + F + f];"),
    ("glu_sigmoid_not_silu", "double silu = gate / (1.0 + exp(-gate));", "double silu = 1.0 / (1.0 + exp(-gate));"),
    ("bf16_truncates", "double n = rint(ldexp(a, -qe));", "double n = trunc(ldexp(a, -qe));"),
    ("bwd_norm_term_sign", "dx[m * K + k] = r * (double)g[k] * dxn[m * K + k] - xv", "dx[m * K + k] = r * (double)g[k] * dxn[m * K + k] + xv"),
    ("bwd_norm_drops_r_cubed", "xv * r * r * r * S / (double)K", "xv * r * S / (double)K"),
    ("bwd_dg_drops_r", "dg[k] += dxn[m * K + k] * xv * r;", "dg[k] += dxn[m * K + k] * xv;"),
    ("bwd_dw_ignores_scale", "((double)q[m * K + k] / (double)s[m])", "(double)q[m * K + k]"),
    ("bwd_dxn_sign_swapped", "a -= (double)dy[m * N + n];", "a += (double)dy[m * N + n];"),
    ("bwd_dxn_drops_gamma", "dxn[m * K + k] = (double)gamma * a;", "dxn[m * K + k] = a;"),
    ("bwd_sum_drops_gain", "S += dxn[m * K + k] * (double)g[k] * (double)orc_bf16_to_float(row[k]);",
     "S += dxn[m * K + k] * (double)orc_bf16_to_float(row[k]);"),
    ("mlgru_forget_from_candidate_rows", "double f = orc_sigmoid(zt[n]);", "double f = orc_sigmoid(zt[d + n]);"),
    ("mlgru_candidate_sigmoid", "double c = orc_silu(zt[d + n]);", "double c = orc_sigmoid(zt[d + n]);"),
    ("mlgru_output_gate_silu", "double g = orc_sigmoid(zt[2 * d + n]);", "double g = orc_silu(zt[2 * d + n]);"),
    ("mlgru_drops_one_minus_f", "h = f * h + (1.0 - f) * c;", "h = f * h + c;"),
    ("mlgru_gate_roles_swapped", "h = f * h + (1.0 - f) * c;", "h = (1.0 - f) * h + f * c;"),
    ("mlgru_no_output_gate", "p[(b * T + t) * d + n] = orc_double_to_bf16(g * h);",
     "p[(b * T + t) * d + n] = orc_double_to_bf16(h);"),
    ("mlgru_state_not_carried_in", "double h = state[b * d + n];", "double h = 0.0;"),
    ("mlgru_state_not_returned", "            state[b * d + n] = h;\n", "            state[b * d + n] += 0.0 * h;\n"),
    ("mlgru_token_stride", "const double* zt = z + (b * T + t) * 3 * d;", "const double* zt = z + (b * T + t) * d;"),
    ("mlgru_out_gain_from_input", "orc_bitlinear_ternary(p, g_out, w_out, gamma_out,", "orc_bitlinear_ternary(p, g_in, w_out, gamma_out,"),
    ("mlgru_master_one_gamma", "float gamma_out = orc_absmean_gamma(W_out, d, d);", "float gamma_out = orc_absmean_gamma(W_in, d, d);"),
    ("layer_glu_reads_x", "orc_glu_ternary(u, g_gu, w_gu, gamma_gu,", "orc_glu_ternary(x, g_gu, w_gu, gamma_gu,"),
    ("layer_drops_first_residual", "u[i] = orc_double_to_bf16((double)orc_bf16_to_float(x[i]) + y[i]);",
     "u[i] = orc_double_to_bf16(y[i]);"),
    ("layer_drops_second_residual", "out[i] = orc_double_to_bf16((double)orc_bf16_to_float(u[i]) + y[i]);",
     "out[i] = orc_double_to_bf16(y[i]);"),
    ("bwd_dw_transposed_token", "a += (double)dy[m * N + n] * ((double)q[m * K + k]", "a += (double)dy[((m + 1) % M) * N + n] * ((double)q[m * K + k]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / "oracle.c"
    mutated.write_text(src.replace(old, new))
    (tmp_path / "oracle.h").write_text(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(lib), str(mutated), "-lm"], check=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), str(lib)],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode != 0, f"mutant {name} survived every pin:\n{res.stdout}\n{res.stderr}"
