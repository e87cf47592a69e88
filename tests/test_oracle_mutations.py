"""Planted mistakes: each entry below copies oracle.c with one plausible error
(a dropped term, a wrong sign or index, a transposed operand ...), builds the
copy with gcc on the CPU, and runs every pin of test_oracle_pins.py against it.
Each planted mistake must fail at least one pin; the unmodified source must
pass them all (test_oracle_pins.py).  Nothing here touches the GPU.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests.test_oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted text)
MUTATIONS = [
    ("resize_keys_a", "const double a = -0.75;", "const double a = -0.5;"),
    ("resize_corners_aligned", "((double)o + 0.5) * (double)Ss / (double)Sd - 0.5",
     "(double)o * (double)(Ss - 1) / (double)(Sd > 1 ? Sd - 1 : 1)"),
    ("resize_border_zero", "idx[m] = i < 0 ? 0 : i > Ss - 1 ? Ss - 1 : i;\n        w[m] = keys_cubic(s - (double)i);",
     "idx[m] = i < 0 ? 0 : i > Ss - 1 ? Ss - 1 : i;\n        w[m] = (i < 0 || i > Ss - 1) ? 0.0 : keys_cubic(s - (double)i);"),
    ("resize_rows_cols", "src[((size_t)iy[m] * Ss + (size_t)ix[n]) * heads + h]",
     "src[((size_t)ix[n] * Ss + (size_t)iy[m]) * heads + h]"),
    ("log_sign", "if (x > 0) return a;", "if (x > 0) return -a;"),
    ("log_base2", "log1p(fabs(x))", "log2(1.0 + fabs(x))"),
    ("relu_dropped", "h[j] = a > 0.0 ? a : 0.0;", "h[j] = a;"),
    ("g_inputs_swapped", "w1[2 * j] * in0 + w1[2 * j + 1] * in1", "w1[2 * j] * in1 + w1[2 * j + 1] * in0"),
    ("b1_dropped", "+ (b1 ? b1[j] : 0.0)", "+ 0.0"),
    ("bias_offset_sign", "(ri - rj + M - 1) * S + (size_t)(ci - cj + M - 1)",
     "(rj - ri + M - 1) * S + (size_t)(cj - ci + M - 1)"),
    ("bias_rows_cols_swapped", "(ri - rj + M - 1) * S + (size_t)(ci - cj + M - 1)",
     "(ci - cj + M - 1) * S + (size_t)(ri - rj + M - 1)"),
    ("bias_dropped", "l += table[", "l += 0.0 * table["),
    ("tau_floor_dropped", "tau[h] > tau_min ? tau[h] : tau_min", "tau[h]"),
    ("shift_direction", "*gi = (wr * M + r + shift) % H;", "*gi = (wr * M + r - shift + H) % H;"),
    ("mask_dropped", "allowed[j] = (char)(region[j] == region[i]);", "allowed[j] = 1;"),
    ("region_off_by_one", "if (p < L - s) return 1;", "if (p <= L - s) return 1;"),
    ("region_first_cut", "if (p < L - M) return 0;", "if (p < L - M - 1) return 0;"),
    ("norm_wrong", "x[e] /= n;", "x[e] /= (n + 1.0);"),
    ("dot_scale", "1.0 / sqrt((double)d)", "1.0 / (double)d"),
    ("rope_sign", "p[1] = x0 * sn + x1 * cs;", "p[1] = x0 * sn - x1 * cs;"),
    ("rope_halves_swapped", "const int pos = half == 0 ? r : c;", "const int pos = half == 0 ? c : r;"),
    ("rope_theta", "pow(base, -(double)k / (double)q4)", "pow(base, -(double)k / (double)(2 * q4))"),
    ("qk_transposed", "s += qs[(size_t)i * d + e] * ks[(size_t)j * d + e];",
     "s += qs[(size_t)j * d + e] * ks[(size_t)i * d + e];"),
    ("v_index", "acc += lg[j] * vs[(size_t)j * d + e];", "acc += lg[j] * vs[(size_t)i * d + e];"),
    ("interleaved_map", "*gi = wr + r * (H / M);", "*gi = wr * M + r;"),
    ("softmax_unnormalised", "for (int j = 0; j < N; ++j) lg[j] /= sum;", ";"),
    ("code_norm_scale", "x / (double)(norm_M - 1) * 8.0", "x / (double)norm_M * 8.0"),
    ("code_norm_base", "log2(1.0 + fabs(u)) / log2(8.0)", "log2(1.0 + fabs(u)) / 3.2"),
    ("code_inputs_paper_order", "*in0 = oracle_code_offset((double)dy, norm_M);\n        *in1 = oracle_code_offset((double)dx, norm_M);",
     "*in0 = oracle_code_offset((double)dx, norm_M);\n        *in1 = oracle_code_offset((double)dy, norm_M);"),
    ("sigmoid_scale", "16.0 / (1.0 + exp(-acc))", "8.0 / (1.0 + exp(-acc))"),
    ("sigmoid_sign", "16.0 / (1.0 + exp(-acc))", "16.0 / (1.0 + exp(acc))"),
    ("bwd_D_dropped", "dr[j] = pr[j] * (dr[j] - Di);", "dr[j] = pr[j] * dr[j];"),
    ("bwd_given_lse_sign", "pr[j] = exp(pr[j] - li);", "pr[j] = exp(li - pr[j]);"),
    ("bwd_given_lse_index", "lse[((size_t)gw * heads + h) * N + i];", "lse[((size_t)gw * heads + h) * N + (N - 1 - i)];"),
    ("bwd_given_D_from_v", "Di += gs[(size_t)i * d + e] * os[(size_t)i * d + e];",
     "Di += gs[(size_t)i * d + e] * vs[(size_t)i * d + e];"),
    ("bwd_dv_index", "gv[(size_t)j * d + e] += pr[j] * gs[(size_t)i * d + e];",
     "gv[(size_t)j * d + e] += pr[j] * gs[(size_t)j * d + e];"),
    ("bwd_norm_projection", "g[e] = (g[e] - xh[e] * proj) / n;", "g[e] = g[e] / n;"),
    ("bwd_rope_not_transposed", "rope_rotate(g, d, -r, -c, f, rope_base);", "rope_rotate(g, d, r, c, f, rope_base);"),
    ("bwd_dtau_sign", "(-1.0 / (tau[h] * tau[h]))", "(1.0 / (tau[h] * tau[h]))"),
    ("bwd_dk_operand", "gk[(size_t)j * d + e] += g * scale * qs[(size_t)i * d + e];",
     "gk[(size_t)j * d + e] += g * scale * ks[(size_t)i * d + e];"),
    ("bwd_table_offset", "my_dtable[((size_t)(ri - rj + M - 1) * S + (size_t)(ci - cj + M - 1)) * heads + h] += g;",
     "my_dtable[((size_t)(rj - ri + M - 1) * S + (size_t)(cj - ci + M - 1)) * heads + h] += g;"),
    ("bwd_mask_dropped", "pr[j] = (region[j] == region[i]) ? l : -INFINITY;",
     "pr[j] = (region[j] == region[i]) ? l : l;"),
    ("cpb_bwd_relu_mask", "const double da = a[j] > 0.0 ? dh : 0.0;", "const double da = dh;"),
    ("cpb_bwd_sigmoid", "dg[o] *= 16.0 * s * (1.0 - s);", "dg[o] *= 16.0 * s;"),
    ("cpb_bwd_inputs_swapped", "dw1[2 * j] += da * in0;", "dw1[2 * j] += da * in1;"),
    ("linear_transposed", "x[t * in + c] * w[(size_t)n * in + c]", "x[t * in + c] * w[(size_t)c * out + n]"),
    ("linear_bias_dropped", "double s = b ? b[n] : 0.0;", "double s = 0.0;"),
    ("ln_unbiased_var", "var /= C;", "var /= (C - 1);"),
    ("ln_eps_outside", "1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    ("ln_resid_dropped", "y[t * C + c] = resid[t * C + c] + gamma[c]", "y[t * C + c] = gamma[c]"),
    ("ln_gamma_beta_swapped", "gamma[c] * (zt[c] - mean) * inv + beta[c]", "beta[c] * (zt[c] - mean) * inv + gamma[c]"),
    ("ln_mean_not_subtracted", "var += (zt[c] - mean) * (zt[c] - mean);", "var += zt[c] * zt[c];"),
    ("dwconv_dy_sign", "const int yy = y + dy, xx = x + dx;", "const int yy = y - dy, xx = x + dx;"),
    ("dwconv_kernel_transposed", "(size_t)(dy + 1) * 3 + (size_t)(dx + 1)]", "(size_t)(dx + 1) * 3 + (size_t)(dy + 1)]"),
    ("dwconv_tap_dropped", "if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue;",
     "if (yy < 0 || yy >= H || xx < 0 || xx >= W || (dy == 1 && dx == 1)) continue;"),
    ("dwconv_bias_dropped", "double s = b ? b[c] : 0.0;", "double s = 0.0;"),
    ("dwconv_overwrites", "out[i] += tmp[i];", "out[i] = tmp[i];"),
    ("v3_shift_t_direction", "(w * M + r + s) % L;", "(w * M + r - s + L) % L;"),
    ("v3_region_t_dropped", "? 9 * axis_region(wt * Mt + t, T, Mt, shift_t) +", "? 0 * axis_region(wt * Mt + t, T, Mt, shift_t) +"),
    ("v3_bias_t_sign", "(size_t)(ti - tj + Mt - 1)", "(size_t)(tj - ti + Mt - 1)"),
    ("v3_dt_input", "w1[3 * j + 2] * in2", "w1[3 * j + 2] * in1"),
    ("v3_interleaved_t", "return part == OR_PART_INTERLEAVED ? w + r * (L / M) : (w * M + r + s) % L;",
     "return part == OR_PART_INTERLEAVED ? w * M + r : (w * M + r + s) % L;"),
    ("lse_max_dropped", "lse[((size_t)wi * heads + h) * N + i] = mx + log(sum);",
     "lse[((size_t)wi * heads + h) * N + i] = log(sum);"),
    ("lse_head_index", "lse[((size_t)wi * heads + h) * N + i] = mx + log(sum);",
     "lse[((size_t)wi * heads + (heads - 1 - h)) * N + i] = mx + log(sum);"),
    ("wl_region_ignored", "if (reg_j != reg_i) continue;", "if (0) continue;"),
    ("wl_A_transposed", "A[((size_t)h * N + i) * N + j]", "A[((size_t)h * N + j) * N + i]"),
    ("wl_bias_index", "bias[(size_t)h * N + i]", "bias[(size_t)h * N + (N - 1 - i)]"),
    ("wl_head_offset", "const double* vj = v + (((size_t)b * H + gi_j) * W + gj_j) * C + (size_t)h * d;",
     "const double* vj = v + (((size_t)b * H + gi_j) * W + gj_j) * C;"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


def test_mutations_are_well_formed():
    src = open(SRC).read()
    for name, old, new in MUTATIONS:
        assert src.count(old) >= 1, f"{name}: text not found in oracle.c"


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(workdir, name, old, new):
    src = open(SRC).read()
    mutant = src.replace(old, new, 1)
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(mutant)
    so = os.path.join(workdir, f"lib{name}.so")
    oracle.build(force=True, src=path, out=so)
    lib = oracle.load(so)
    # the first pin that fails is enough; the pin that imports transformers
    # (seconds) runs last
    order = sorted(PINS, key=lambda n: n == "cpb_released_code")
    caught = None
    for pin_name in order:
        try:
            PINS[pin_name](lib)
        except (AssertionError, ValueError):
            caught = pin_name
            break
    assert caught, f"planted mistake {name} passed every pin"
