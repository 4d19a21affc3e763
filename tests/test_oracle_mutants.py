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

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

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
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    pattern, repl = MUTANTS[name]
    src = open(SRC).read()
    assert pattern in src, f"mutant {name}: pattern no longer in the oracle"
    mutated = src.replace(pattern, repl)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
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
