"""Each plausible mistake planted in a copy of the oracle fails a pin.

The copy is compiled on the CPU into a temporary directory; the real oracle
source is never modified.
"""

import os

import pytest

import oracle
import pins

MUTANTS = {
    "lambda_sign": ("p1[j] - lam * p2[j]", "p1[j] + lam * p2[j]"),
    "lambda_drop_init": ("exp(dot1) - exp(dot2) + lambda_init", "exp(dot1) - exp(dot2)"),
    "lambda_swap_terms": ("exp(dot1) - exp(dot2)", "exp(dot2) - exp(dot1)"),
    "lambda_init_schedule": ("-0.3 * (double)(depth - 1)", "-0.3 * (double)depth"),
    "causal_ignored": ("return causal ? i + 1 : n;", "return causal ? n : n;"),
    "causal_strict": ("return causal ? i + 1 : n;", "return causal ? (i > 0 ? i : 1) : n;"),
    "decode_alignment_top_left": ("causal ? nk - nq + i + 1 : nk", "causal ? nq - nq + i + 1 : nk"),
    "decode_alignment_off_by_one": ("causal ? nk - nq + i + 1 : nk", "causal ? nk - nq + i : nk"),
    "decode_keys_from_query_offsets": ("cu_k[s], nkeys, h, H, Hkv", "cu_q[s], nkeys, h, H, Hkv"),
    "rope_sign": ("out[2 * j] = x0 * c - x1 * sn;", "out[2 * j] = x0 * c + x1 * sn;"),
    "rope_pairs_half_apart": ("const double x0 = (double)x[2 * j], x1 = (double)x[2 * j + 1];",
                              "const double x0 = (double)x[j], x1 = (double)x[j + d / 2];"),
    "rope_global_positions": ("t, t - a, a,", "t, t, a,"),
    "rope_key_position_zero": ("row_rot(k + (((ka + j) * Hkv + g) * 2 + map) * (int64_t)d, d, rp, j, kd);",
                               "row_rot(k + (((ka + j) * Hkv + g) * 2 + map) * (int64_t)d, d, rp, 0, kd);"),
    "rope_table_row_stride": ("rp->cos + pos * (int64_t)(d / 2)", "rp->cos + pos * (int64_t)d"),
    "rope_bf16_rounding_dropped": ("    if (rp->round_bf16)\n", "    if (0)\n"),
    "bwd_softmax_no_D": ("const double ds = p[m][j] * (dpj - D);", "const double ds = p[m][j] * dpj;"),
    "bwd_map2_lambda_sign": ("dO[1][c] = -lam[h] * dp;", "dO[1][c] = lam[h] * dp;"),
    "bwd_rmsnorm_no_r3_term": ("const double dp = r * gc - r * r * r * pre[c] * gp / (double)dv2;",
                               "const double dp = r * gc;"),
    "bwd_dv_from_map1_only": ("dvr[c] += p[m][j] * dO[m][c];", "dvr[c] += p[0][j] * dO[0][c];"),
    "bwd_dq_from_q": ("dqr[c] += scale * ds * (double)kr[c];", "dqr[c] += scale * ds * (double)qr[c] + 0.0 * kr[c];"),
    "bwd_dk_unscaled": ("dkr[c] += scale * ds * (double)qr[c];", "dkr[c] += ds * (double)qr[c];"),
    "bwd_dw_without_r": ("tdw[task * dv2 + c] += (double)dyr[c] * pre[c] * r * (1.0 - lambda_init);",
                         "tdw[task * dv2 + c] += (double)dyr[c] * pre[c] * (1.0 - lambda_init);"),
    "bwd_dlambda_sign": ("dl -= dp * o[1][c];", "dl += dp * o[1][c];"),
    "bwd_dlq1_wrong_vector": ("dlq1[off + c] = dlam * ea * (double)lk1[off + c];",
                              "dlq1[off + c] = dlam * ea * (double)lq1[off + c];"),
    "bwd_dlk2_sign": ("dlk2[off + c] = -dlam * eb * (double)lq2[off + c];",
                      "dlk2[off + c] = dlam * eb * (double)lq2[off + c];"),
    "gqa_modulo": ("h / (H / Hkv)", "h % Hkv"),
    "scale_full_width": ("1.0 / sqrt((double)d)", "1.0 / sqrt(2.0 * d)"),
    "scale_squared": ("1.0 / sqrt((double)d)", "1.0 / (double)d"),
    "eps_dropped": ("ss / (double)dv + eps", "ss / (double)dv"),
    "rms_sum_not_mean": ("ss / (double)dv + eps", "ss + eps"),
    "final_scale_dropped": ("* wc * (1.0 - lambda_init)", "* wc"),
    "weight_ignored": ("w ? (double)w[c] : 1.0", "1.0"),
    "k_map_swapped": ("+ g) * 2 + map) * (int64_t)d", "+ g) * 2 + (1 - map)) * (int64_t)d"),
    "q_map_swapped": ("((qt * H + h) * 2 + map)", "((qt * H + h) * 2 + (1 - map))"),
    "key_row_is_query_row": ("k + (((ka + j) * Hkv", "k + (((qt) * Hkv"),
    "v_uses_query_head": ("((ka + j) * Hkv + g) * (int64_t)dv", "((ka + j) * Hkv + h % Hkv) * (int64_t)dv"),
    "softmax_no_max_shift": ("exp(p[j] - mx)", "exp(p[j])"),
    "softmax_wrong_normaliser": ("p[j] /= z;", "p[j] /= (double)nkeys;"),
    "per_head_lambda_offset": ("const int64_t o = (int64_t)h * stride;", "const int64_t o = 0 * stride;"),
    "per_head_lambda_index": ("diff_row(q, k, v, lam[h],", "diff_row(q, k, v, lam[0],"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    path = os.path.join(tmp_path, "mut.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib_path = oracle.build(path, os.path.join(tmp_path, f"libmut_{name}.so"))
    lib = oracle.load(lib_path)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
