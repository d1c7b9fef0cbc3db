"""Negative controls for the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's source,
builds it with g++ into a temporary directory, and requires that at least one
pin of tests/oracle_pins.py fails on it.  A pin suite that a dropped term, a
wrong sign or index, a swapped nibble or a wrong tie rule can slip through
would not be worth trusting."""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = {
    "nibble_order": ("codes[2 * j] | (codes[2 * j + 1] << 4)", "codes[2 * j + 1] | (codes[2 * j] << 4)"),
    "drop_eps": ("ss / (double)H + (double)eps", "ss / (double)H"),
    "mean_over_H_minus_1": ("ss / (double)H + (double)eps", "ss / (double)(H - 1) + (double)eps"),
    "fp8_max_240": ("(float)amax / 448.0f", "(float)amax / 240.0f"),
    "e8m0_off_by_one": ("std::ilogb(amax) - 2 + 127", "std::ilogb(amax) - 1 + 127"),
    "e4m3_ties_away": ("int quantum_exp = (e < -6) ? -9 : e - 3;\n  double r = std::ldexp(std::nearbyint(",
                       "int quantum_exp = (e < -6) ? -9 : e - 3;\n  double r = std::ldexp(std::round("),
    "e4m3_subnormal_spacing": ("(e < -6) ? -9 : e - 3", "(e < -7) ? -10 : e - 3"),
    "e4m3_no_saturation": ("if (a > 448.0) a = 448.0;  // saturate (Inf included)", ""),
    "e2m1_ties_away": ("int quantum_exp = (e < 0) ? -1 : e - 1;\n  double r = std::ldexp(std::nearbyint(",
                       "int quantum_exp = (e < 0) ? -1 : e - 1;\n  double r = std::ldexp(std::round("),
    "bf16_ties_away": ("double n = std::nearbyint(std::ldexp(a, -quantum_exp));  // ties to even",
                       "double n = std::round(std::ldexp(a, -quantum_exp));"),
    "residual_sign": ("e.value(x[i]) + e.value(res[i])", "e.value(x[i]) - e.value(res[i])"),
    "norm_reads_unrounded_sum": (
        "    double v = e.value(r[i]);\n    ss += v * v;",
        "    double v = e.value(x[i]) + e.value(res[i]);\n    ss += v * v;"),
    "weight_index_reversed": ("e.value(r[i]) * rstd * e.value(w[i])",
                              "e.value(r[i]) * rstd * e.value(w[H - 1 - i])"),
    "f16_subnormal_quantum": ("(e < -14) ? -24 : e - 10", "(e < -14) ? -25 : e - 10"),
    "f16_saturates_instead_of_inf": ("if (r > 65504.0) return (uint16_t)(sign | 0x7C00);",
                                     "if (r > 65504.0) return (uint16_t)(sign | 0x7BFF);"),
    "f16_exponent_bias": ("return s * std::ldexp(1.0 + m / 1024.0, e - 15);", "return s * std::ldexp(1.0 + m / 1024.0, e - 14);"),
    "zero_sign_dropped": ("q[i] = std::signbit(v) ? 0x80 : 0x00;", "q[i] = 0x00;"),
    "gemma_without_one": ("(1.0 + bf16_value(w[i]))", "bf16_value(w[i])"),
    "qk_interleave_stride": ("qg + t * ld_qg + 2 * D * h", "qg + t * ld_qg + D * h"),
    "qk_gate_offset": ("const uint16_t* gate_part = q_part + D;", "const uint16_t* gate_part = q_part + D + 1;"),
    "quotient_by_reciprocal": ("float quotient = (float)v / s;", "float quotient = (float)v * (1.0f / s);"),
    "qk_fp8_granule_per_token": ("quantize_fp8_rows(kBf16, q_bf16.data(), T * Hq, D, D, q_codes, q_scale)",
                                 "quantize_fp8_rows(kBf16, q_bf16.data(), T, Hq * D, Hq * D, q_codes, q_scale)"),
    "tscale_row_major_index": ("scale_out[g * ld_scale + m] = row_major[m * G + g]",
                               "scale_out[m * G + g] = row_major[m * G + g]"),
    "qk_mxfp4_k_from_q": ("quantize_mxfp4_rows(kBf16, k_bf16.data(), T * Hk, D, k_codes, k_scale)",
                          "quantize_mxfp4_rows(kBf16, q_bf16.data(), T * Hk, D, k_codes, k_scale)"),
    "mxfp4_scale_direction": ("std::ldexp(e.value(y[i]), -((int)b - 127))", "std::ldexp(e.value(y[i]), ((int)b - 127))"),
    "group_scale_index": ("scale_out + m * G + g);", "scale_out + m * G);"),
    "amax_ignores_nan": ("    if (std::isnan(a)) return a;\n", ""),
    "quotient_in_double": ("float quotient = (float)v / s;  // IEEE fp32 division\n      q[i] = e4m3fn_round((double)quotient);",
                           "double quotient = v / (double)s;\n      q[i] = e4m3fn_round(quotient);"),
    "sum_of_squares_in_float": ("double ss = 0.0;", "float ss = 0.0f;"),
    "qk_drop_eps": ("std::sqrt(ss / (double)D + (double)eps)", "std::sqrt(ss / (double)D)"),
    "qk_mean_over_D_minus_1": ("std::sqrt(ss / (double)D + (double)eps)", "std::sqrt(ss / (double)(D - 1) + (double)eps)"),
    "qk_k_uses_q_weight": ("gemma_norm(k + t * ld_k + D * h, k_w,", "gemma_norm(k + t * ld_k + D * h, q_w,"),
    "qk_fp8_k_from_q": ("quantize_fp8_rows(kBf16, k_bf16.data(), T * Hk, D, D, k_codes, k_scale)",
                        "quantize_fp8_rows(kBf16, q_bf16.data(), T * Hk, D, D, k_codes, k_scale)"),
}


def _failing_pins(lib_path):
    ref = oracle.Oracle(lib_path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(ref)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as exc:  # a crash of the broken oracle also counts as caught
            failed.append(f"{pin.__name__}: {type(exc).__name__}")
    return failed


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # a broken oracle may make NaN from an overflow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    original, mutated = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(original) >= 1, f"mutation target not found in the oracle: {original!r}"
    path = os.path.join(tmp_path, "rq_oracle.cpp")
    with open(path, "w") as f:
        f.write(src.replace(original, mutated))
    os.symlink(os.path.join(os.path.dirname(oracle.SOURCE), "rq_oracle.h"), os.path.join(tmp_path, "rq_oracle.h"))
    lib = oracle.build(source=path, output=os.path.join(tmp_path, f"librq_{name}.so"))
    failed = _failing_pins(lib)
    assert failed, f"no pin caught the planted mistake {name!r}"
