"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the oracle's pins fail for each one: evidence that the pins are tight
enough to catch a dropped term, a wrong sign or index, or a transposed
operand."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_int4.py", "tests/test_oracle_requant.py",
             "tests/test_oracle_gemm.py", "tests/test_oracle_conv.py",
             "tests/test_oracle_dwconv.py", "tests/test_oracle_quant.py",
             "tests/test_oracle_zp.py", "tests/test_oracle_f16.py"]

MUTANTS = {
    "nibble_order": ("(i % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
                     "(i % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "no_sign_extension": ("return code < 8 ? code : code - 16;", "return code;"),
    "no_rounding_term": ("return 2 * r >= unit ? q + 1 : q;", "return q;"),
    "ties_rounded_down": ("return 2 * r >= unit ? q + 1 : q;", "return 2 * r > unit ? q + 1 : q;"),
    "truncating_division": ("if (r < 0) {", "if (0) {"),
    "rounding_unit_doubled": ("const __int128 unit = (__int128)1 << s;",
                              "const __int128 unit = (__int128)1 << (s + 1);"),
    "saturation_low": ("round_half_up_pow2((__int128)x * mult, shift), -128, 127)",
                       "round_half_up_pow2((__int128)x * mult, shift), -127, 127)"),
    "bias_dropped": ("const int64_t x = acc + bias;\n    if (x < INT32_MIN || x > INT32_MAX)\n"
                     "        return ORC_E_RANGE;\n    if (shift < 1 || shift > 63 || mult < 0)\n",
                     "const int64_t x = acc;\n    if (x < INT32_MIN || x > INT32_MAX)\n"
                     "        return ORC_E_RANGE;\n    if (shift < 1 || shift > 63 || mult < 0)\n"),
    "bias_after_multiply": ("*out = saturate(round_half_up_pow2((__int128)x * mult, shift)",
                            "*out = saturate(round_half_up_pow2((__int128)acc * mult + bias, shift)"),
    "k_reversed": ("acc += (int64_t)a[k] * (int64_t)b[k];",
                   "acc += (int64_t)a[k] * (int64_t)b[K - 1 - k];"),
    "k_dropped_term": ("for (int64_t k = 0; k < K; ++k)\n        acc += (int64_t)a[k] * (int64_t)b[k];",
                       "for (int64_t k = 0; k + 1 < K; ++k)\n        acc += (int64_t)a[k] * (int64_t)b[k];"),
    "conv_pad_offset": ("int64_t ih = oh * sh - ph + kh;", "int64_t ih = oh * sh + kh;"),
    "conv_weight_transposed": ("Wt[((oc * KH + kh) * KW + kw) * C_in + ci]",
                               "Wt[((oc * KW + kw) * KH + kh) * C_in + ci]"),
    "conv_out_size": ("return span / stride + 1;", "return span / stride;"),
    "dw_pad_offset": ("const int64_t ih = oh * sh + kh - ph;", "const int64_t ih = oh * sh + kh;"),
    "dw_weight_layout": ("Wt[(kh * KW + kw) * C + c]", "Wt[c * KH * KW + kh * KW + kw]"),
    "dw_channel_mix": ("X[((b * H + ih) * W + iw) * C + c]",
                       "X[((b * H + ih) * W + iw) * C + (c + 1) % C]"),
    "quant_half_even": ("int64_t r = (int64_t)f + ((a - f) >= 0.5f ? 1 : 0);",
                        "int64_t r = (int64_t)f + ((a - f) > 0.5f ? 1 : 0);"),
    "quant_qmax_int4": ("const float qmax = bits == 4 ? 7.0f : 127.0f;",
                        "const float qmax = bits == 4 ? 8.0f : 127.0f;"),
    "quant_clip_inverted": ("const float sc = amax / (qmax / clip_ratio);",
                            "const float sc = amax / (qmax * clip_ratio);"),
    "quant_signed_max": ("float a = v < 0 ? -v : v;\n            if (a > amax)",
                         "float a = v;\n            if (a > amax)"),
    "quant_nibble_swap": ("if (k % 2 == 0)\n                    *byte",
                          "if (k % 2 == 1)\n                    *byte"),
    "zp_out_zero_dropped": ("saturate(y + out_zero, act_min, act_max)",
                            "saturate(y, act_min, act_max)"),
    "zp_out_zero_after_clamp": ("*out = saturate(y + out_zero, act_min, act_max);",
                                "*out = (int8_t)(saturate(y, act_min, act_max) + out_zero);"),
    "act_clamp_ignored": ("saturate(y + out_zero, act_min, act_max)",
                          "saturate(y + out_zero, -128, 127)"),
    "zp_a_zero_dropped": ("acc += ((int64_t)a[k] - za) * ((int64_t)b[k] - zb);",
                          "acc += ((int64_t)a[k]) * ((int64_t)b[k] - zb);"),
    "zp_b_zero_sign": ("acc += ((int64_t)a[k] - za) * ((int64_t)b[k] - zb);",
                       "acc += ((int64_t)a[k] - za) * ((int64_t)b[k] + zb);"),
    "zp_conv_pad_zero": ("int64_t x = inside ? X[((b * H + y) * W + xx) * C_in + ci] : za;",
                         "int64_t x = inside ? X[((b * H + y) * W + xx) * C_in + ci] : 0;"),
    "zp_dw_pad_zero": ("const int64_t x = inside ? X[(((b * H) + y) * W + xx) * C + c] : za;",
                       "const int64_t x = inside ? X[(((b * H) + y) * W + xx) * C + c] : 0;"),
    "zp_dw_w_zero_dropped": ("const int64_t w = Wt[t * C + c];\n        acc += (x - za) * (w - zb);",
                             "const int64_t w = Wt[t * C + c];\n        acc += (x - za) * w;"),
    "msb_nibble_order": ("const int code = (i % 2 == 0) ? (byte >> 4) : (byte & 0x0F);",
                         "const int code = (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);"),
    "f16_ties_up": ("if (rem > half || (rem == half && (r & 1u)))", "if (rem >= half)"),
    "f16_truncate": ("if (rem > half || (rem == half && (r & 1u)))", "if (0)"),
    "f16_scale_b_dropped": ("            if (scale_b)\n                t = t * scale_b[n];",
                            "            if (scale_b)\n                t = t;"),
    "f16_overflow_check_dropped": ("if (a >= 0x477FF000u)", "if (0)"),
    "s4s4_operand_repeated": ("orc_int4_at(a, k) * (int64_t)orc_int4_at(b, k)",
                              "orc_int4_at(a, k) * (int64_t)orc_int4_at(a, k)"),
    "s8s4_k_reversed": ("acc += (int64_t)a[k] * (int64_t)orc_int4_at(b, k);",
                        "acc += (int64_t)a[k] * (int64_t)orc_int4_at(b, K - 1 - k);"),
    "s4_row_stride_in_bytes": ("(const uint8_t *)A + m * (lda / 2)", "(const uint8_t *)A + m * lda"),
    "requant_shift_per_tensor": ("dot_any(ka, A, lda, m, kb, B, ldb, n, K);\n"
                                 "            if (acc < INT32_MIN || acc > INT32_MAX)\n"
                                 "                status |= ORC_E_RANGE;\n            int8_t y = 0;\n"
                                 "            status |= orc_requant(acc, bias ? bias[n] : 0, mult[n], shift[n]",
                                 "dot_any(ka, A, lda, m, kb, B, ldb, n, K);\n"
                                 "            if (acc < INT32_MIN || acc > INT32_MAX)\n"
                                 "                status |= ORC_E_RANGE;\n            int8_t y = 0;\n"
                                 "            status |= orc_requant(acc, bias ? bias[n] : 0, mult[n], shift[0]"),
    "gemm_range_check_dropped": ("dot_any(ka, A, lda, m, kb, B, ldb, n, K);\n"
                                 "            if (acc < INT32_MIN || acc > INT32_MAX)\n"
                                 "                status |= ORC_E_RANGE;\n            int8_t y = 0;",
                                 "dot_any(ka, A, lda, m, kb, B, ldb, n, K);\n            int8_t y = 0;"),
    "msb_range_check_dropped": ("(int64_t)a[k] * (int64_t)orc_int4_at_msb(b, k);\n            if (acc < INT32_MIN || acc > INT32_MAX)\n"
                                "                status |= ORC_E_RANGE;\n",
                                "(int64_t)a[k] * (int64_t)orc_int4_at_msb(b, k);\n"),
    "conv_stride_axes_swapped": ("int64_t ih = oh * sh - ph + kh;", "int64_t ih = oh * sw - ph + kh;"),
    "conv_pixel_row_index": ("int64_t oh = (p / Wo) % Ho;\n        int64_t ow = p % Wo;\n"
                             "        for (int64_t oc = 0; oc < C_out; ++oc) {\n"
                             "            int64_t acc = conv_acc_at(",
                             "int64_t oh = (p / Ho) % Ho;\n        int64_t ow = p % Wo;\n"
                             "        for (int64_t oc = 0; oc < C_out; ++oc) {\n"
                             "            int64_t acc = conv_acc_at("),
    "f16_subnormal_shift": ("shift = -e - 1;", "shift = -e - 2;"),
    "f16_underflow_threshold": ("if (e < -25)", "if (e < -24)"),
    "f16_nan_as_infinity": ("(a > 0x7F800000u ? 0x7E00u : 0x7C00u)", "(0x7C00u)"),
    "f16_scale_a_by_position": ("t = t * scale_a[m];", "t = t * scale_a[r];"),
    "f16_decode_subnormal_unit": ("v = (float)m * (1.0f / 16777216.0f);", "v = (float)m * (1.0f / 8388608.0f);"),
    "f16_decode_bias": ("((uint32_t)(e - 15 + 127) << 23)", "((uint32_t)(e - 14 + 127) << 23)"),
    "bf16_decode_shift": ("{(uint32_t)b << 16}", "{(uint32_t)b << 15}"),
    "quant_low_clamp": ("q = -(int64_t)qmax;", "q = -(int64_t)qmax - 1;"),
    "quant_scale_stored_inverse": ("scale[m] = sc;", "scale[m] = sc > 0.0f ? 1.0f / sc : 0.0f;"),
    "quant_int4_row_stride": ("(uint8_t *)Q + m * (ldq / 2) + k / 2", "(uint8_t *)Q + m * (ldq / 4) + k / 2"),
    "quant_int8_row_stride": ("((int8_t *)Q)[m * ldq + k]", "((int8_t *)Q)[m * (ldq / 2) + k]"),
    "dw_tap_dropped": ("for (int64_t kw = 0; kw < KW; ++kw) {\n            const int64_t iw",
                       "for (int64_t kw = 0; kw + 1 < KW; ++kw) {\n            const int64_t iw"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    src = open(os.path.join(ROOT, "oracle", "qgemm_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    msrc = tmp_path / "qgemm_oracle.c"
    msrc.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(msrc),
                    "-o", str(lib)], check=True)
    env = dict(os.environ, QG_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


def test_unmutated_copy_passes(tmp_path):
    lib = tmp_path / "liboracle_copy.so"
    oracle.build(out=str(lib))
    env = dict(os.environ, QG_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]


def test_ubsan_build_runs_clean(tmp_path):
    """The oracle built with UBSan (trap on any undefined behaviour, e.g. a
    signed int64 overflow in the requantize) passes the pins."""
    lib = tmp_path / "liboracle_ubsan.so"
    oracle.build(extra_flags=["-fsanitize=undefined", "-fno-sanitize-recover=all"],
                 out=str(lib))
    env = dict(os.environ, QG_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_requant.py", "tests/test_oracle_conv.py",
                        "tests/test_oracle_zp.py", "tests/test_oracle_f16.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
