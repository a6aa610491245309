"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake (a dropped term, a wrong sign, a wrong index, a
swapped operand, a missing rounding) in a temporary copy of the C oracle,
builds it with gcc, and runs the pin tests against that build in a child
process.  The pins pass on the real oracle, so every mutant must make at
least one of them fail.  Nothing here touches the GPU.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qknr_oracle.c")

MUTANTS = {
    "eps_outside_root": ("return 1.0 / sqrt(ms + eps);", "return 1.0 / (sqrt(ms) + eps);"),
    "mean_over_D_minus_1": ("double ms = ss / (double)D;", "double ms = ss / (double)(D - 1);"),
    "rotation_sign_first": ("y[i] = n[i] * c[i] - n[i + h] * s[i];",
                            "y[i] = n[i] * c[i] + n[i + h] * s[i];"),
    "rotation_sign_second": ("y[i + h] = n[i + h] * c[i] + n[i] * s[i];",
                             "y[i + h] = n[i + h] * c[i] - n[i] * s[i];"),
    "rotation_sense_both": ("y[i] = n[i] * c[i] - n[i + h] * s[i];\n        y[i + h] = n[i + h] * c[i] + n[i] * s[i];",
                            "y[i] = n[i] * c[i] + n[i + h] * s[i];\n        y[i + h] = n[i + h] * c[i] - n[i] * s[i];"),
    "interleaved_pairs": ("y[i] = n[i] * c[i] - n[i + h] * s[i];\n        y[i + h] = n[i + h] * c[i] + n[i] * s[i];",
                          "y[2*i] = n[2*i] * c[i] - n[2*i + 1] * s[i];\n        y[2*i + 1] = n[2*i + 1] * c[i] + n[2*i] * s[i];"),
    "freq_missing_factor_2": ("return pow(theta, -2.0 * (double)i / (double)denom);",
                              "return pow(theta, -1.0 * (double)i / (double)denom);"),
    "freq_reversed_index": ("return pow(theta, -2.0 * (double)i / (double)denom);",
                            "return pow(theta, -2.0 * (double)(denom / 2 - 1 - i) / (double)denom);"),
    "no_fp32_rounding_of_cos": ("c[i] = (double)(float)(attn * cos(phi));", "c[i] = attn * cos(phi);"),
    "weight_reversed": ("n[j] = w[j] * (x[j] - m) * r;", "n[j] = w[D - 1 - j] * (x[j] - m) * r;"),
    "tail_unnormalised": ("for (int j = R; j < D; ++j)\n        y[j] = n[j];",
                          "for (int j = R; j < D; ++j)\n        y[j] = x[j];"),
    "k_uses_q_weight": ("oracle_fwd_row(k + off, wk, bk, c, s, D, R, eps, flags, yk + off);",
                        "oracle_fwd_row(k + off, wq, bk, c, s, D, R, eps, flags, yk + off);"),
    "token_index_as_position": ("oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row",
                                "oracle_rope_cos_sin_gen(t, theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row"),
    "head_offset_transposed": ("int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row",
                               "int64_t off = (hd * tokens + t) * (int64_t)D;\n            oracle_fwd_row"),
    "bwd_transpose_sign": ("g[i] = dy[i] * c[i] + dy[i + h] * s[i];", "g[i] = dy[i] * c[i] - dy[i + h] * s[i];"),
    "bwd_forward_rotation_instead_of_transpose": (
        "g[i] = dy[i] * c[i] + dy[i + h] * s[i];\n        g[i + h] = dy[i + h] * c[i] - dy[i] * s[i];",
        "g[i] = dy[i] * c[i] - dy[i + h] * s[i];\n        g[i + h] = dy[i + h] * c[i] + dy[i] * s[i];"),
    "bwd_dropped_mean_term": ("dx[j] = r * (u[j] - mu - xh[j] * mean);", "dx[j] = r * (u[j] - mu);"),
    "bwd_missing_r": ("dx[j] = r * (u[j] - mu - xh[j] * mean);", "dx[j] = (u[j] - mu - xh[j] * mean);"),
    "bwd_dw_uses_raw_x": ("dw[j] += g[j] * xh[j];", "dw[j] += g[j] * x[j];"),
    "bwd_dw_uses_dy": ("dw[j] += g[j] * xh[j];", "dw[j] += dy[j] * xh[j];"),
    "bwd_mean_weightless": ("u[j] = w[j] * g[j];\n        dot += u[j] * xh[j];",
                            "u[j] = w[j] * g[j];\n        dot += g[j] * xh[j];"),
    "bf16_ties_away": ("double m = nearbyint(a / quantum);", "double m = round(a / quantum);"),
    "bf16_truncate": ("double m = nearbyint(a / quantum);", "double m = floor(a / quantum);"),
    # convention variants
    "interleaved_sign_even": ("y[2 * i] = n[2 * i] * c[i] - n[2 * i + 1] * s[i];",
                              "y[2 * i] = n[2 * i] * c[i] + n[2 * i + 1] * s[i];"),
    "interleaved_sign_odd": ("y[2 * i + 1] = n[2 * i + 1] * c[i] + n[2 * i] * s[i];",
                             "y[2 * i + 1] = n[2 * i + 1] * c[i] - n[2 * i] * s[i];"),
    "interleaved_as_half_split": (
        "y[2 * i] = n[2 * i] * c[i] - n[2 * i + 1] * s[i];\n        y[2 * i + 1] = n[2 * i + 1] * c[i] + n[2 * i] * s[i];",
        "y[i] = n[i] * c[i] - n[i + h] * s[i];\n        y[i + h] = n[i + h] * c[i] + n[i] * s[i];"),
    "interleaved_flag_ignored_fwd": ("if (flags & ORACLE_INTERLEAVED)\n        oracle_rotate_interleaved(n",
                                     "if (0)\n        oracle_rotate_interleaved(n"),
    "interleaved_flag_ignored_bwd": ("if (flags & ORACLE_INTERLEAVED)\n        oracle_rotate_interleaved_t(",
                                     "if (0)\n        oracle_rotate_interleaved_t("),
    "interleaved_bwd_sign": ("g[2 * i] = dy[2 * i] * c[i] + dy[2 * i + 1] * s[i];",
                             "g[2 * i] = dy[2 * i] * c[i] - dy[2 * i + 1] * s[i];"),
    "interleaved_bwd_forward_rotation": (
        "g[2 * i] = dy[2 * i] * c[i] + dy[2 * i + 1] * s[i];\n        g[2 * i + 1] = dy[2 * i + 1] * c[i] - dy[2 * i] * s[i];",
        "g[2 * i] = dy[2 * i] * c[i] - dy[2 * i + 1] * s[i];\n        g[2 * i + 1] = dy[2 * i + 1] * c[i] + dy[2 * i] * s[i];"),
    "freq_head_dim_ignored_fwd": (
        "int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;\n    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];\n    for (int64_t t = 0; t < tokens; ++t) {\n        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row",
        "int denom = R;\n    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];\n    for (int64_t t = 0; t < tokens; ++t) {\n        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row"),
    "freq_head_dim_half_fwd": (
        "int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;\n    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];\n    for (int64_t t = 0; t < tokens; ++t) {\n        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row",
        "int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D / 2 : R;\n    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];\n    for (int64_t t = 0; t < tokens; ++t) {\n        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_fwd_row"),
    # QK-LayerNorm, biases, frequency tables
    "ln_mean_not_subtracted": ("n[j] = w[j] * (x[j] - m) * r;", "n[j] = w[j] * x[j] * r;"),
    "ln_variance_uncentred": ("ss += (x[j] - m) * (x[j] - m);", "ss += x[j] * x[j];"),
    "ln_mean_over_D_minus_1": ("m = sx / (double)D;", "m = sx / (double)(D - 1);"),
    "ln_bwd_missing_mean_u": ("double mu = (flags & ORACLE_LAYERNORM) ? su / (double)D : 0.0;",
                              "double mu = 0.0;"),
    "ln_bwd_xh_uncentred": ("xh[j] = (x[j] - m) * r;", "xh[j] = x[j] * r;"),
    "bias_sign": ("n[j] += b[j];", "n[j] -= b[j];"),
    "bias_dropped": ("if (b)\n        for (int j = 0; j < D; ++j)\n            n[j] += b[j];", ""),
    "bias_after_weight_on_raw_x": ("n[j] += b[j];", "n[j] += b[j] * x[j];"),
    "db_uses_dy": ("db[j] += g[j];", "db[j] += dy[j];"),
    "db_scaled_by_w": ("db[j] += g[j];", "db[j] += w[j] * g[j];"),
    "freq_table_ignored": ("double f = freq ? freq[i] : oracle_inv_freq(theta, i, denom);",
                           "double f = oracle_inv_freq(theta, i, denom);"),
    "attention_factor_on_cos_only": ("s[i] = (double)(float)(attn * sin(phi));",
                                     "s[i] = (double)(float)sin(phi);"),
    "attention_factor_ignored": ("c[i] = (double)(float)(attn * cos(phi));\n        s[i] = (double)(float)(attn * sin(phi));",
                                 "c[i] = (double)(float)cos(phi);\n        s[i] = (double)(float)sin(phi);"),
    "freq_head_dim_ignored_bwd": (
        "int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;\n    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];\n    for (int64_t t = 0; t < tokens; ++t) {\n        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_bwd_row",
        "int denom = R;\n    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];\n    for (int64_t t = 0; t < tokens; ++t) {\n        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);\n        for (int hd = 0; hd < hq; ++hd) {\n            int64_t off = (t * hq + hd) * (int64_t)D;\n            oracle_bwd_row"),
    # norm groups and per-head weights
    "group_stats_over_one_head": ("double r = oracle_row_stats(x, g * D, eps, flags, &m);",
                                  "double r = oracle_row_stats(x, D, eps, flags, &m);"),
    "group_bwd_stats_over_one_head": ("double r = oracle_row_stats(x, L, eps, flags, &m);",
                                      "double r = oracle_row_stats(x, D, eps, flags, &m);"),
    "group_head_weight_not_strided": ("double v = w[hd * wstride + j] * (x[hd * D + j] - m) * r;",
                                      "double v = w[j] * (x[hd * D + j] - m) * r;"),
    "group_bias_not_strided": ("v += b[hd * wstride + j];", "v += b[j];"),
    "group_rotates_first_head_only": ("oracle_rotate_half_split(nh, c, s, R, yh);",
                                      "oracle_rotate_half_split(n, c, s, R, yh);"),
    "group_bwd_mean_over_D": ("double mean = dot / (double)L;", "double mean = dot / (double)D;"),
    "group_bwd_ln_mean_u_over_D": ("double mu = (flags & ORACLE_LAYERNORM) ? su / (double)L : 0.0;",
                                   "double mu = (flags & ORACLE_LAYERNORM) ? su / (double)D : 0.0;"),
    "group_bwd_u_weight_not_strided": ("u[e] = w[hd * wstride + j] * gg[e];", "u[e] = w[j] * gg[e];"),
    "group_dw_not_strided": ("dw[hd * wstride + j] += gg[e] * xh[e];", "dw[j] += gg[e] * xh[e];"),
    "group_db_uses_dy": ("db[hd * wstride + j] += gg[e];", "db[hd * wstride + j] += dy[e];"),
    "group_q_uses_k_group_size": (
        "oracle_fwd_group(q + off, wq + h0 * ws, bq ? bq + h0 * ws : 0, ws, c, s, gq, D, R, eps,",
        "oracle_fwd_group(q + off, wq + h0 * ws, bq ? bq + h0 * ws : 0, ws, c, s, gk, D, R, eps,"),
    "group_bwd_dw_head_offset_dropped": (
        "scratch, scratch + L, scratch + 2 * L, dq + off, dwq + h0 * ws,",
        "scratch, scratch + L, scratch + 2 * L, dq + off, dwq,"),
    # Best-Fit-Decreasing packing
    "bfd_worst_fit": ("if (capacity - fill[b] >= L && (best < 0 || fill[b] > fill[best]))",
                      "if (capacity - fill[b] >= L && (best < 0 || fill[b] < fill[best]))"),
    "bfd_first_fit": ("if (capacity - fill[b] >= L && (best < 0 || fill[b] > fill[best]))",
                      "if (capacity - fill[b] >= L && best < 0)"),
    "bfd_tie_highest_index": ("if (capacity - fill[b] >= L && (best < 0 || fill[b] > fill[best]))",
                              "if (capacity - fill[b] >= L && (best < 0 || fill[b] >= fill[best]))"),
    "bfd_unstable_sort": ("while (j > 0 && len[order[j - 1]] < len[i]) {",
                          "while (j > 0 && len[order[j - 1]] <= len[i]) {"),
    "bfd_increasing_order": ("while (j > 0 && len[order[j - 1]] < len[i]) {",
                             "while (j > 0 && len[order[j - 1]] > len[i]) {"),
    "bfd_fit_off_by_one": ("if (capacity - fill[b] >= L && (best < 0 || fill[b] > fill[best]))",
                           "if (capacity - fill[b] > L && (best < 0 || fill[b] > fill[best]))"),
    "bfd_positions_from_one": ("pos[doc_start[i] + t] = t;", "pos[doc_start[i] + t] = t + 1;"),
    "bfd_no_filler_segment": ("seg += ndoc[b] + (fill[b] < capacity ? 1 : 0);", "seg += ndoc[b];"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not found exactly once" % name
    path = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    with open(path, "w") as fh:
        fh.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-o", lib,
                    path, "-lm"], check=True)
    env = dict(os.environ, QKNR_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        names = sorted(MUTANTS)
        with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
            results = dict(zip(names, ex.map(lambda n: _run_mutant(n, tmp), names)))
    survivors = [n for n, (rc, _) in results.items() if rc == 0]
    assert not survivors, "mutants not caught by any pin: %s" % survivors
    # a collection error or crash is not a caught mutant
    bad = [n for n, (rc, out) in results.items() if rc not in (1,)]
    assert not bad, {n: results[n][1] for n in bad}
