"""The pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of oracle.c (a dropped term, a
wrong sign, index, shift or nibble half, a transposed operand), builds it
with gcc into a temporary library and checks that at least one pin fails.
CPU only; the oracle's own build is never touched.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "q4_1_min_sign": ("w[j] = d * (double)q + m;", "w[j] = d * (double)q - m;"),
    "q4_1_min_offset": ("double d = half_at(b), m = half_at(b + 2);", "double d = half_at(b), m = half_at(b + 4);"),
    "q4_1_codes_at_2": ("const uint8_t *qs = b + 4;\n    for (int j = 0; j < 32; j++) {\n        int q = (j < 16) ? (qs[j] & 15) : (qs[j - 16] >> 4);\n        w[j] = d * (double)q + m;",
                        "const uint8_t *qs = b + 2;\n    for (int j = 0; j < 32; j++) {\n        int q = (j < 16) ? (qs[j] & 15) : (qs[j - 16] >> 4);\n        w[j] = d * (double)q + m;"),
    "q4_0_offset": ("w[j] = d * (double)(q - 8);", "w[j] = d * (double)(q - 7);"),
    "q4_0_nibble_halves": ("(j < 16) ? (qs[j] & 15) : (qs[j - 16] >> 4);\n        w[j] = d * (double)(q - 8);",
                           "(j < 16) ? (qs[j] >> 4) : (qs[j - 16] & 15);\n        w[j] = d * (double)(q - 8);"),
    "q4_1_nibble_halves": ("(j < 16) ? (qs[j] & 15) : (qs[j - 16] >> 4);\n        w[j] = d * (double)q + m;",
                           "(j < 16) ? (qs[j] >> 4) : (qs[j - 16] & 15);\n        w[j] = d * (double)q + m;"),
    "q8_0_unsigned": ("(double)(int8_t)b[2 + j]", "(double)(uint8_t)b[2 + j]"),
    "q8_0_off_by_one": ("(int8_t)b[2 + j]", "(int8_t)b[1 + j]"),
    "q4_k_scale_mask": ("*sc = s[i] & 63;", "*sc = s[i] & 31;"),
    "q4_k_high_bits": ("*sc = (s[i + 4] & 15) | ((s[i - 4] >> 6) << 4);", "*sc = (s[i + 4] & 15) | ((s[i - 4] >> 6) << 5);"),
    "q4_k_min_from_scale_byte": ("*mn = (s[i + 4] >> 4) | ((s[i] >> 6) << 4);", "*mn = (s[i + 4] >> 4) | ((s[i - 4] >> 6) << 4);"),
    "q4_k_min_sign": ("(double)q - dmin * (double)mn", "(double)q + dmin * (double)mn"),
    "q5_k_min_sign": ("(hi << 4)) - dmin * (double)mn", "(hi << 4)) + dmin * (double)mn"),
    "q4_k_nibble_parity": ("int q = (i % 2 == 0) ? (byte & 15) : (byte >> 4);", "int q = (i % 2 == 1) ? (byte & 15) : (byte >> 4);"),
    "q4_k_chunk": ("uint8_t byte = qs[(i / 2) * 32 + e];\n        int q =", "uint8_t byte = qs[(i % 4) * 32 + e];\n        int q ="),
    "q5_k_chunk": ("uint8_t byte = qs[(i / 2) * 32 + e];\n            int lo =", "uint8_t byte = qs[(i % 4) * 32 + e];\n            int lo ="),
    "q5_k_fifth_bit": ("int hi = (qh[e] >> i) & 1;", "int hi = (qh[e] >> (i / 2)) & 1;"),
    "q5_k_fifth_bit_weight": ("(double)(lo | (hi << 4))", "(double)(lo | (hi << 3))"),
    "q5_k_qh_offset": ("*qh = b + 16, *qs = b + 48;", "*qh = b + 16, *qs = b + 44;"),
    "q6_k_nibble_groups": ("int lo4 = (g < 2) ?", "int lo4 = (g < 1) ?"),
    "q6_k_qh_shift": ("(qh[32 * h + l] >> (2 * g)) & 3", "(qh[32 * h + l] >> g) & 3"),
    "q6_k_ql_half": ("ql[64 * h + 32 * (g & 1) + l]", "ql[32 * h + 32 * (g & 1) + l]"),
    "q6_k_subscale": ("sc[j / 16]", "sc[j / 32]"),
    "q6_k_offset": ("(double)(q - 32)", "(double)(q - 31)"),
    "half_exponent": ("ldexp((double)(1024 + frac), expo - 25)", "ldexp((double)(1024 + frac), expo - 24)"),
    "half_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "row_offset": ("blob + m * nb * bb", "blob + m * nb * (bb - 2)"),
    "transposed_x": ("const float *x = X + n * K;", "const float *x = X + n;"),
    "dropped_term": ("for (int64_t k = 0; k < K; k++) {", "for (int64_t k = 1; k < K; k++) {"),
    "magnitude_signed": ("mag += fabs(p);", "mag += p;"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "silu_no_factor": ("return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    "swiglu_swapped": ("double o = oracle_silu(g[i]) * u[i];", "double o = oracle_silu(u[i]) * g[i];"),
    "swiglu_gate_twice": ("rc = oracle_matmul_rows(dtype, up, M, K, N, X, nrows, rows, tmp, u, su);",
                          "rc = oracle_matmul_rows(dtype, gate, M, K, N, X, nrows, rows, tmp, u, su);"),
    "argmax_last_tie": ("if (bi < 0 || y64[m] > y64[bi]) bi = m;", "if (bi < 0 || y64[m] >= y64[bi]) bi = m;"),
    "argmax_min": ("if (bi < 0 || y64[m] > y64[bi]) bi = m;", "if (bi < 0 || y64[m] < y64[bi]) bi = m;"),
    "argmax_skips_last": ("for (int64_t m = 0; m < M; m++) {\n            if (y64[m] != y64[m]) continue;",
                          "for (int64_t m = 0; m + 1 < M; m++) {\n            if (y64[m] != y64[m]) continue;"),
    "q8a_ties_away": ("float q = rintf(v[t] * id);", "float q = roundf(v[t] * id);"),
    "q8a_unrounded_scale": ("scales[n * nb + b] = (float)oracle_half_to_double(oracle_float_to_half(d));",
                            "scales[n * nb + b] = d;"),
    "q8a_codes_from_f16_scale": ("float r = 1.0f / d;", "float r = 1.0f / (float)oracle_half_to_double(oracle_float_to_half(d));"),
    "q8a_signed_max": ("float a = fabsf(v[t]);", "float a = v[t];"),
    "q8a_no_finite_guard": ("float id = (d != 0.0f && isfinite(r)) ? r : 0.0f;", "float id = (d != 0.0f) ? r : 0.0f;"),
    "q8a_nan_code": ("if (isnan(q)) c = 0;", "if (isnan(q)) c = 127;"),
    "q8a_divide_by_128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q8a_first_block_scale": ("(double)scales[n * nb32 + j / 32]", "(double)scales[n * nb32]"),
    "q8a_sum_drops_first": ("for (int64_t j = 0; j < K; j++) {", "for (int64_t j = 1; j < K; j++) {"),
    "q8a_token0_codes": ("(double)quants[n * K + j]", "(double)quants[j]"),
    "q8a_splus_no_offset": ("magp += (fabs(w[j] - o[j]) + fabs(o[j])) * fabs(xq);", "magp += fabs(w[j]) * fabs(xq);"),
    "q8a_offset_sign": ("for (int e = 0; e < 32; e++) o[32 * i + e] = -(dmin * (double)mn);",
                        "for (int e = 0; e < 32; e++) o[32 * i + e] = (dmin * (double)mn);"),
    "q8a_q4_1_offset_missing": ("for (int j = 0; j < 32; j++) o[j] = m;", "for (int j = 0; j < 32; j++) o[j] = 0.0 * m;"),
    "half_ties_away": ("double m = rint(ldexp(a, 11 - E));", "double m = round(ldexp(a, 11 - E));"),
    "half_overflow_threshold": ("if (a >= 65520.0) return", "if (a >= 65504.0) return"),
    "half_subnormal_truncates": ("rint(ldexp(a, 24))", "floor(ldexp(a, 24))"),
    "half_exponent_bias": ("int e = E - 1 + 15;", "int e = E + 15;"),
    "f32_rounding": ("Y[n * nrows + r] = (float)acc;", "Y[n * nrows + r] = (float)(acc * (1.0 + 0x1p-23));"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(source.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(src), "-o", str(lib), "-lm"],
                   check=True)
    L = oracle.load_variant(str(lib))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(L)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"
