"""Plant plausible mistakes in copies of the oracle and require that the pins
catch every one.  Each mutant is the oracle's C source with one textual edit,
built with gcc into a temporary directory on the CPU."""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "tq_oracle.c")

# (name, [(old, new), ...]); every `old` must occur in the source
MUTANTS = [
    ("msb_first_slots", [("c << (2 * (k % 4))", "c << (6 - 2 * (k % 4))"),
                         ("byte >> (2 * (k % 4))", "byte >> (6 - 2 * (k % 4))")]),
    ("code_map_sign", [("c = v + 1;", "c = 1 - v;"), ("(int8_t)(c - 1)", "(int8_t)(1 - c)")]),
    ("binary_bit_map", [("b = (v + 1) / 2;", "b = (1 - v) / 2;"),
                        ("(int8_t)(2 * b - 1)", "(int8_t)(1 - 2 * b)")]),
    ("dropped_first_term", [("for (int64_t j = 0; j < group; j++)",
                             "for (int64_t j = 1; j < group; j++)")]),
    ("scale_first_group_only", [("scales[n * G + g]", "scales[n * G]")]),
    ("scale_transposed", [("scales[n * G + g]", "scales[g * N + n]")]),
    ("x_group_offset_dropped", [("x[m * K + g * group + j]", "x[m * K + j]")]),
    ("t_group_stride", [("t[g * group + j]", "t[g * 64 + j]")]),
    ("half_exponent_bias", [("e - 25", "e - 24")]),
    ("half_subnormal", [("ldexp((double)f, -24)", "ldexp((double)f, -25)")]),
    ("bound_signed", [("apart += fabs(tx);", "apart += tx;")]),
    ("scale_abs_missing", [("bound += fabs(s) * apart;", "bound += s * apart;")]),
    ("row_stride", [("codes + n * row_bytes", "codes + n * (row_bytes / 2)")]),
    ("accept_code3", [("if (c == 3) {", "if (c == 4) {")]),
    ("embed_row_stride", [("codes + id * row_bytes", "codes + id * (row_bytes / 2)")]),
    ("embed_scale_row", [("scales[id * G + k / group]", "scales[k / group]")]),
    ("embed_scale_group", [("scales[id * G + k / group]", "scales[id * G]")]),
    ("embed_out_row", [("out[i * K + k]", "out[k]")]),
    ("t5_msb_digit_first", [("int value = 0, power = 1;", "int value = 0, power = 81;"),
                            ("power *= 3;", "power /= 3;")]),
    ("t5_group_stride", [("codes[n * rb + 26 * g + b] = (uint8_t)value;",
                          "codes[n * rb + 25 * g + b] = (uint8_t)value;")]),
    ("t5_no_row_padding", [("return (raw + 15) / 16 * 16;", "return raw;")]),
    ("t5_tail_digits_unchecked", [("else if (c != 0)", "else if (c > 2)")]),
    ("t5_range_unchecked", [("if (value != 0) {", "if (value > 1) {")]),
    ("affine_bias_dropped", [("double w = sg * (double)q[k] + bg;", "double w = sg * (double)q[k];")]),
    ("affine_bias_group", [("double bg = oracle_half_to_double(biases[n * G + k / group]);",
                            "double bg = oracle_half_to_double(biases[n * G]);")]),
    ("affine_level_mask", [("t[n * K + k] = (int8_t)((byte >> (2 * (k % 4))) & 3);",
                            "t[n * K + k] = (int8_t)((byte >> (2 * (k % 4))) & 1);")]),
    ("affine_bound_bias", [("+ fabs(bg) * fabs(x[m * K + k]);", ";")]),
    ("kv_amax_divisor", [("uint16_t d = oracle_float_to_half(amax / 7.0f);",
                          "uint16_t d = oracle_float_to_half(amax / 8.0f);")]),
    ("kv_nibble_offset", [("nib[v * 256 + 32 * g + j] = (uint8_t)(q + 8);",
                           "nib[v * 256 + 32 * g + j] = (uint8_t)(q + 7);")]),
    ("kv_round_truncates", [("float r = rintf((float)oracle_half_to_double(xg[j]) / df);",
                             "float r = truncf((float)oracle_half_to_double(xg[j]) / df);")]),
    ("half_round_ties_up", [("if (rem > half || (rem == half && (q & 1u))) q++;",
                             "if (rem >= half) q++;")]),
    ("attn_scale", [("s[t] = dot / 16.0;", "s[t] = dot / 8.0;")]),
    ("attn_gqa_map", [("int64_t kvh = h / rep;", "int64_t kvh = h % n_kv;")]),
    ("attn_group_of_dim", [("((double)kn[j] - 8.0) * oracle_half_to_double(kd[j / 32]);",
                            "((double)kn[j] - 8.0) * oracle_half_to_double(kd[j / 16 % 8]);")]),
    ("attn_v_scale", [("oracle_half_to_double(vs[(kvh * T + t) * 8 + j / 32]);",
                       "oracle_half_to_double(vs[(kvh * T + t) * 8]);")]),
    # a hand-made row split that drops the remainder rows when the thread
    # count does not divide N (single-threaded runs are unaffected)
    ("omp_split_drops_rows", [("#include <math.h>", "#include <math.h>\n#include <omp.h>"),
                              ("#pragma omp for schedule(static)\n        for (int64_t n = 0; n < N; n++) {\n            if (!t) continue;",
                               "for (int64_t n = omp_get_thread_num() * (N / omp_get_num_threads()); "
                               "n < (omp_get_thread_num() + 1) * (N / omp_get_num_threads()); n++) {\n"
                               "            if (!t) continue;")]),
    ("omp_split_drops_rows_affine", [("#include <math.h>", "#include <math.h>\n#include <omp.h>"),
                                     ("#pragma omp for schedule(static)\n        for (int64_t n = 0; n < N; n++) {\n            if (!q) continue;",
                                      "for (int64_t n = omp_get_thread_num() * (N / omp_get_num_threads()); "
                                      "n < (omp_get_thread_num() + 1) * (N / omp_get_num_threads()); n++) {\n"
                                      "            if (!q) continue;")]),
    ("t5_code_map", [("t[n * K + 128 * g + 5 * b + i] = (int8_t)(c - 1);",
                      "t[n * K + 128 * g + 5 * b + i] = (int8_t)(1 - c);"),
                     ("value += (t[n * K + 128 * g + 5 * b + i] + 1) * power;",
                      "value += (1 - t[n * K + 128 * g + 5 * b + i]) * power;")]),
]


def _build_mutant(tmp_path, name, edits):
    with open(SRC) as f:
        text = f.read()
    for old, new in edits:
        assert old in text, (name, old)
        text = text.replace(old, new)
    src = tmp_path / ("%s.c" % name)
    src.write_text(text)
    lib_path = str(tmp_path / ("lib%s.so" % name))
    oracle.build(lib_path, src=str(src))
    return oracle.load(lib_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, edits):
    lib = _build_mutant(tmp_path, name, edits)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(lib)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, "no pin caught mutant %s" % name
