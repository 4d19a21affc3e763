"""Strength of the oracle's pins: plant a plausible mistake in a copy of the oracle
source (on the CPU), build it, and check that the pin battery rejects it.

Each mutant is one edit of attn_oracle.c; the pattern must occur in the source so
that a refactor of the oracle cannot silently turn a mutant into a no-op.
"""
import os
import subprocess

import pytest

import oracle
from tests import pins

ORACLE_DIR = os.path.dirname(oracle.__file__)
SRC = os.path.join(ORACLE_DIR, "attn_oracle.c")
QSRC = os.path.join(ORACLE_DIR, "fp8_quant_oracle.c")
BSRC = os.path.join(ORACLE_DIR, "attn_bwd_oracle.c")

MUTANTS = {
    "gqa_map_modulo": ("h / group", "h % Hkv"),
    "causal_excludes_diagonal": ("hi = causal ? i : N - 1;", "hi = causal ? i - 1 : N - 1;"),
    "causal_one_extra_key": ("hi = causal ? i : N - 1;", "hi = causal ? (i + 1 < N ? i + 1 : i) : N - 1;"),
    "window_left_off_by_one": ("if (left >= 0 && i - left > lo) lo = i - left;",
                               "if (left >= 0 && i - left + 1 > lo) lo = i - left + 1;"),
    "window_right_one_extra": ("if (right >= 0 && i + right < hi) hi = i + right;",
                               "if (right >= 0 && i + right + 1 < hi) hi = i + right + 1;"),
    "window_sides_swapped": ("if (left >= 0 && i - left > lo) lo = i - left;",
                             "if (right >= 0 && i - right > lo) lo = i - right;"),
    "window_right_ignored": ("if (right >= 0 && i + right < hi) hi = i + right;", ""),
    "window_overrides_causal": ("if (right >= 0 && i + right < hi) hi = i + right;",
                                "if (right >= 0) hi = i + right < N - 1 ? i + right : N - 1;"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale_squared": ("s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    "max_not_subtracted": ("const double e = exp(s[j] - m);", "const double e = exp(s[j]);"),
    "exp_sign_flipped": ("const double e = exp(s[j] - m);", "const double e = exp(m - s[j]);"),
    "lse_base2": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "lse_drops_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "no_normalisation": ("for (int t = 0; t < d; ++t) o_row[t] /= l;", ""),
    "dot_drops_last_dim": ("for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];",
                           "for (int t = 0; t + 1 < d; ++t) dot += qi[t] * kj[t];"),
    "v_rows_reversed": ("const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;",
                        "const double* vj = v + (((size_t)b * N + (jlo + jhi - j)) * Hkv + hk) * d;"),
    "k_used_for_v": ("const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;",
                     "const double* vj = k + (((size_t)b * N + j) * Hkv + hk) * d;"),
    "f16_exponent_bias": ("mag = ldexp((double)(1024 + f), e - 25);", "mag = ldexp((double)(1024 + f), e - 24);"),
    "bf16_exponent_bias": ("mag = ldexp((double)(128 + f), e - 134);", "mag = ldexp((double)(128 + f), e - 133);"),
    "e4m3_subnormal_scale": ("mag = ldexp((double)f, -9);", "mag = ldexp((double)f, -10);"),
    "e4m3_ieee_style_top_exponent": ("if (e == 15 && f == 7) mag = NAN;", "if (e == 15) mag = NAN;"),
    "decode_ignores_descale": ("dst[i] = x * mult;", "dst[i] = x;"),
    "kv_causal_top_left": ("const int pos = Nk - Nq + i;", "const int pos = i;"),
    "kv_causal_one_short": ("const int pos = Nk - Nq + i;", "const int pos = Nk - Nq + i - 1;"),
    "block_key_index_shifted": ("keep[j] = row[j / block] != 0", "keep[j] = row[(j + 1) / block] != 0"),
    "block_query_index_shifted": ("+ i / block) * nb;", "+ (i + 1 < N ? i + 1 : i) / block) * nb;"),
    "block_mask_heads_ignored": ("(mask_heads == 1 ? 0 : h)", "0"),
    "block_causal_ignored": ("!= 0 && (!causal || j <= i);", "!= 0;"),
    "block_empty_row_unguarded": ("if (m == -INFINITY) {                      /* no visible key */",
                                  "if (0) {"),
    # the single-row entry points
    "rows_window_dropped": ("key_range(i, N, causal, left, right, &jlo, &jhi);\n      attn_row(qi, k, v, Hkv, N, d, "
                            "jlo, jhi, scale, b, h / group, s, o_rows",
                            "key_range(i, N, causal, -1, -1, &jlo, &jhi);\n      attn_row(qi, k, v, Hkv, N, d, "
                            "jlo, jhi, scale, b, h / group, s, o_rows"),
    "rows_gqa_modulo": ("jlo, jhi, scale, b, h / group, s, o_rows", "jlo, jhi, scale, b, h % Hkv, s, o_rows"),
    "rows_gathered_query_reversed": ("q_is_rows ? q + (size_t)r * d :", "q_is_rows ? q + (size_t)(nrows - 1 - r) * d :"),
    "rows_lse_slot_shifted": ("lse_rows + r);", "lse_rows + (r + 1) % nrows);"),
    "block_rows_causal_dropped": ("block_keep(mask, mask_heads, block, N, causal, h, i, keep);\n      "
                                  "attn_row_keep(qi, k, v, Hkv, N, d, keep, scale, b, h / group, s, o_rows",
                                  "block_keep(mask, mask_heads, block, N, 0, h, i, keep);\n      "
                                  "attn_row_keep(qi, k, v, Hkv, N, d, keep, scale, b, h / group, s, o_rows"),
}

# mutants of the block-quantisation oracle (fp8_quant_oracle.c)
QMUTANTS = {
    "encode_ties_away": ("double m = rint(ldexp(a, 3 - E));", "double m = round(ldexp(a, 3 - E));"),
    "encode_subnormal_quantum": ("code = (uint8_t)rint(a * 512.0);", "code = (uint8_t)rint(a * 256.0);"),
    "encode_no_saturation": ("if (a > 448.0) a = 448.0;", ""),
    "encode_drops_sign": ("return neg ? (uint8_t)(code | 0x80) : code;", "return code;"),
    "fwht_sign_swapped": ("x[j + h] = a - b;", "x[j + h] = b - a;"),
    "fwht_skips_last_stage": ("for (int h = 1; h < d; h <<= 1)", "for (int h = 1; 2 * h < d; h <<= 1)"),
    "exponent_strict_bound": ("<= 448.0 ? E - 8 : E - 7;", "< 448.0 ? E - 8 : E - 7;"),
    "exponent_one_too_high": ("<= 448.0 ? E - 8 : E - 7;", "<= 448.0 ? E - 7 : E - 6;"),
    "exponent_no_floor": ("if (e < -127) e = -127;", ""),
    "signs_ignored": ("y[t] = signs ? (float)xr[t] * signs[t] : (float)xr[t];", "y[t] = (float)xr[t];"),
    "amax_signed": ("if (fabsf(y[t]) > amax) amax = fabsf(y[t]);", "if (y[t] > amax) amax = y[t];"),
    "scale_not_applied": ("c[t] = oracle_e4m3_encode((float)ldexp((double)y[t], -e));",
                          "c[t] = oracle_e4m3_encode(y[t]);"),
}


# mutants of the gradient oracle (attn_bwd_oracle.c)
BMUTANTS = {
    "bwd_D_without_p": ("D += p[j] * s;", "D += s;"),
    "bwd_dS_sign": ("const double ds = p[j] * (dp[j] - D);", "const double ds = p[j] * (D - dp[j]);"),
    "bwd_dK_unscaled": ("dkj[t] += scale * ds * qi[t];", "dkj[t] += ds * qi[t];"),
    "bwd_dV_uses_dS": ("dvj[t] += p[j] * gi[t];", "dvj[t] += ds * gi[t];"),
    "bwd_dQ_uses_q": ("dqi[t] += scale * ds * kj[t];", "dqi[t] += scale * ds * qi[t];"),
    "bwd_gqa_modulo": ("const int hk = h / group;", "const int hk = h % Hkv;"),
    "bwd_P_unnormalised": ("for (int j = jlo; j <= jhi; ++j) p[j] /= l;", ""),
    "bwd_dP_uses_k": ("const double* vj = v + (((size_t)b * N + j) * Hkv + hk) * d;",
                      "const double* vj = k + (((size_t)b * N + j) * Hkv + hk) * d;"),
    "bwd_window_left_off_by_one": ("if (left >= 0 && i - left > lo) lo = i - left;",
                                   "if (left >= 0 && i - left + 1 > lo) lo = i - left + 1;"),
    # the key-row gradient and the absolute-value sums
    "dkdv_rows_causal_from_zero": ("for (int i = causal ? j : 0; i < N; ++i) {", "for (int i = 0; i < N; ++i) {"),
    "dkdv_rows_causal_skips_diagonal": ("for (int i = causal ? j : 0; i < N; ++i) {",
                                        "for (int i = causal ? j + 1 : 0; i < N; ++i) {"),
    "dkdv_rows_lse_unscaled": ("const double p = exp(scale * s - lse[row]);", "const double p = exp(s - lse[row]);"),
    "dkdv_rows_D_dropped": ("const double ds = p * (dp - D[row]);", "const double ds = p * dp;"),
    "dkdv_rows_one_head": ("for (int h = hk * group; h < (hk + 1) * group; ++h)", "for (int h = hk * group; h == hk * group; ++h)"),
    "dkdv_rows_dv_from_q": ("dvj[t] += p * gi[t];", "dvj[t] += p * qi[t];"),
    "dkdv_mag_signed": ("m1[t] += fabs(ds) * fabs(qi[t]);", "m1[t] += ds * fabs(qi[t]);"),
    "dkdv_mag_weight_dropped": ("m1[d + t] += p * w[row] * fabs(qi[t]);", "m1[d + t] += p * fabs(qi[t]);"),
    "dq_mag_p_signed_k": ("m2[t] += p[j] * fabs(kj[t]);", "m2[t] += p[j] * kj[t];"),
}

ALL = {**{n: (SRC,) + m for n, m in MUTANTS.items()}, **{n: (QSRC,) + m for n, m in QMUTANTS.items()},
       **{n: (BSRC,) + m for n, m in BMUTANTS.items()}}


@pytest.mark.parametrize("name", sorted(ALL))
def test_mutant_is_caught(name, tmp_path):
    target, pattern, repl = ALL[name]
    sources = []
    for path in (SRC, QSRC, BSRC):
        src = open(path).read()
        if path == target:
            assert pattern in src, f"mutant {name}: pattern no longer in the oracle"
            src = src.replace(pattern, repl)
        c_path = tmp_path / os.path.basename(path)
        c_path.write_text(src)
        sources.append(str(c_path))
    so_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-ffp-contract=off", "-o",
                    str(so_path), *sources, "-lm"], check=True)
    lib = oracle.load(str(so_path))
    saved = oracle._lib()
    oracle._LIB = lib
    failures = []
    try:
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError) as e:
                failures.append(pin.__name__)
    finally:
        oracle._LIB = saved
    assert failures, f"mutant {name} passed every pin"
