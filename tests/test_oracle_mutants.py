"""Planted mistakes in a copy of the oracle must each fail a pin.

Every mutant is a plausible slip (a dropped term, a wrong sign, divisor,
index or rounding rule) applied textually to a temporary copy of
oracle/dquant_oracle.c, compiled with the oracle's own flags and run
against the pins in oracle_pins.py.  The real oracle is never modified.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins

SRC = oracle.SOURCE

MUTANTS = [
    ("sym_divisor_scale_opt", "float sc = amax / offset_opt;", "float sc = amax / scale_opt;"),
    ("asym_offset_sign", "float off = offset_opt - q_hi;", "float off = q_hi - offset_opt;"),
    ("asym_offset_subtracted", "float t = q + off;", "float t = q - off;"),
    ("asym_range_uses_max_only", "float range = hi - lo;", "float range = hi;"),
    ("asym_qhi_from_min", "float q_hi = hi / sc;", "float q_hi = lo / sc;"),
    ("round_half_away", "float r = nearbyintf(t);", "float r = roundf(t);"),
    ("nan_to_low", "if (isnan(t))\n        return 0;", "if (isnan(t))\n        return lo;"),
    ("int4_nibble_order",
     "yr[k] = (uint8_t)((c[2 * k] & 0xF) | ((c[2 * k + 1] & 0xF) << 4));",
     "yr[k] = (uint8_t)((c[2 * k + 1] & 0xF) | ((c[2 * k] & 0xF) << 4));"),
    ("int32_word_order", "<< (4 * i);", "<< (4 * (7 - i));"),
    ("expert_le", "if (r < (int64_t)gi[e])", "if (r <= (int64_t)gi[e])"),
    ("expert_tail_first", "return n_experts - 1;\n}", "return 0;\n}"),
    ("smooth_row_index", "s = smooth + e * n;", "s = smooth + e;"),
    ("smooth_divides", "v[j] = s ? xv * s[j] : xv;", "v[j] = s ? xv / s[j] : xv;"),
    ("absmax_no_abs", "float a = fabsf(v[j]);", "float a = v[j];"),
    ("ada_unbiased_var", "double var = ss / (double)H;", "double var = ss / (double)(H - 1);"),
    ("ada_no_eps", "double rstd = 1.0 / sqrt(var + eps);", "double rstd = 1.0 / sqrt(var);"),
    ("ada_modulate_without_one", "double yv = ln * (1.0 + sc) + sh;", "double yv = ln * sc + sh;"),
    ("ada_shift_dropped", "double yv = ln * (1.0 + sc) + sh;", "double yv = ln * (1.0 + sc);"),
    ("ada_bias_times_weight", "double ln = (xv - mean) * rstd * w + bb;",
     "double ln = ((xv - mean) * rstd + bb) * w;"),
    ("ada_smooth_dropped", "yv = yv * (double)load_as_f32(smooth, smooth_dtype, j);", "yv = yv;"),
    ("ada_batch_index", "double sc = (double)load_as_f32(scale, scale_dtype, b * H + j);",
     "double sc = (double)load_as_f32(scale, scale_dtype, j);"),
    ("ada_divisor_128", "float qs = amax / 127.0f;", "float qs = amax / 128.0f;"),
    ("aq_offset_sign", "float u = v + o;", "float u = v - o;"),
    ("aq_group_mod", "p = i * ((n + group_size - 1) / group_size) + j / group_size;",
     "p = i * ((n + group_size - 1) / group_size) + j % group_size;"),
    ("aq_group_floor_count", "p = i * ((n + group_size - 1) / group_size) + j / group_size;",
     "p = i * (n / group_size) + j / group_size;"),
    ("aq_kdim0_index", "p = (i / group_size) * n + j;", "p = (i % group_size) * n + j;"),
    ("aq_channel_is_token", "else if (policy == ORC_PER_CHANNEL)\n                p = j;",
     "else if (policy == ORC_PER_CHANNEL)\n                p = i;"),
    ("bf16_ties_up", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))",
     "if (lower >= 0x8000u)"),
    ("f16_subnormal_quantum", "double q = nearbyint(ldexp(a, 24));",
     "double q = nearbyint(ldexp(a, 23));"),
    ("f16_trunc", "double q = nearbyint(ldexp(a, 10 - E));", "double q = floor(ldexp(a, 10 - E));"),
    ("e4m3_bias8", "v = ldexp((double)(8 + f), e - 10);", "v = ldexp((double)(8 + f), e - 11);"),
    ("e4m3_no_subnormal", "v = ldexp((double)f, -9);", "v = 0.0;"),
    ("e5m2_bias16", "v = ldexp((double)(4 + f), e - 17);", "v = ldexp((double)(4 + f), e - 18);"),
    ("e5m2_no_inf", "return f ? nanf(\"\") : (sign ? -INFINITY : INFINITY);", "return nanf(\"\");"),
    ("e2m1_high_nibble_first", "return orc_e2m1_to_f32((uint8_t)((i & 1) ? byte >> 4 : byte & 0xF));",
     "return orc_e2m1_to_f32((uint8_t)((i & 1) ? byte & 0xF : byte >> 4));"),
    ("e2m1_subnormal_one", "v = 0.5 * f;", "v = 1.0 * f;"),
    ("e2m1_bias2", "v = ldexp((double)(2 + f), e - 2);", "v = ldexp((double)(2 + f), e - 3);"),
    ("e8m0_bias128", "return (float)ldexp(1.0, (int)b - 127);", "return (float)ldexp(1.0, (int)b - 128);"),
    ("bf16_widen_shift", "return bits_to_f32((uint32_t)h << 16);",
     "return bits_to_f32((uint32_t)h << 15);"),
    ("mx_e4m3_emax_7", "f.maxv = 448.0; f.emax = 8;", "f.maxv = 448.0; f.emax = 7;"),
    ("mx_e2m1_emax_3", "f.maxv = 6.0; f.emax = 2;", "f.maxv = 6.0; f.emax = 3;"),
    ("mx_e5m2_saturates_to_inf", "f.maxv = 57344.0;", "f.maxv = 65536.0;"),
    ("mx_ceil_log2", "shared = (e - 1) - f.emax;", "shared = e - f.emax;"),
    ("mx_no_saturation", "if (v > f.maxv)\n        v = f.maxv;", "if (v > 2 * f.maxv)\n        v = f.maxv;"),
    ("mx_round_half_away", "double q = nearbyint(ldexp(a, f.mbits - E));",
     "double q = round(ldexp(a, f.mbits - E));"),
    ("mx_subnormal_quantum", "if (E < emin)\n        E = emin; /* the subnormals share",
     "if (E < emin - 1)\n        E = emin - 1; /* the subnormals share"),
    ("f64_half_subnormal_quantum", "if (E < emin)\n        E = emin;\n    double q = nearbyint(ldexp(a, mbits - E)); /* quanta",
     "if (E < emin - 1)\n        E = emin - 1;\n    double q = nearbyint(ldexp(a, mbits - E)); /* quanta"),
    ("mx_fp4_nibble_order", "uint8_t* b = (uint8_t*)y + i / 2;\n        if (i & 1)",
     "uint8_t* b = (uint8_t*)y + i / 2;\n        if (!(i & 1))"),
    ("mx_clamp_fp32_min", "if (shared < -127)\n                    shared = -127;",
     "if (shared < -126)\n                    shared = -126;"),
    ("mx_inf_not_flagged", "if (!isfinite(v))\n                    finite = 0;",
     "if (isnan(v))\n                    finite = 0;"),
    ("mx_zero_sign_dropped", "unsigned sign = signbit(t) ? 1u << (f.bits - 1) : 0u;",
     "unsigned sign = t < 0 ? 1u << (f.bits - 1) : 0u;"),
    ("mx_scale_floor_count", "int64_t si = axis == 1 ? o * blocks + j : j * n + o;",
     "int64_t si = axis == 1 ? o * (along / gs) + j : j * n + o;"),
    ("mx_axis0_scale_index", "int64_t si = axis == 1 ? o * blocks + j : j * n + o;",
     "int64_t si = axis == 1 ? o * blocks + j : o * blocks + j;"),
    ("wq_offset_subtracted", "float u = v + load_as_f32(offset, param_dtype, p);",
     "float u = v - load_as_f32(offset, param_dtype, p);"),
    ("wq_group_index_transposed", "p = transpose_x2 ? nn * groups + kk / group_size : (kk / group_size) * n + nn;",
     "p = nn * groups + kk / group_size;"),
    ("wq_int4_unsigned", "return v >= 8 ? v - 16 : v;", "return v;"),
    ("wq_int4_high_first", "int v = (i & 1) ? byte >> 4 : byte & 0xF;", "int v = (i & 1) ? byte & 0xF : byte >> 4;"),
    ("wq_weight_layout_ignored", "int64_t i = transpose_x2 ? nn * k + kk : kk * n + nn;", "int64_t i = kk * n + nn;"),
    ("wq_bf16_truncated", "W[kk * n + nn] = param_dtype == ORC_BF16 ? orc_f32_to_bf16(t) : orc_f32_to_f16(t);",
     "W[kk * n + nn] = param_dtype == ORC_BF16 ? (uint16_t)(f32_to_bits(t) >> 16) : orc_f32_to_f16(t);"),
    ("wq_bias_dropped", "acc += (double)load_as_f32(bias, x_dtype, nn);", "acc += 0.0;"),
    ("wq_x3_dropped", "acc += (double)load_as_f32(x3, x_dtype, mm * n + nn);", "acc += 0.0;"),
    ("wq_x1_row_index", "double a = (double)load_as_f32(x1, x_dtype, mm * k + kk);",
     "double a = (double)load_as_f32(x1, x_dtype, kk);"),
    ("f64_half_via_f32", "    double a = fabs(x);\n    if (isinf(x))\n        return (uint16_t)(sign | inf);",
     "    double a = fabs((double)(float)x);\n    if (isinf(x))\n        return (uint16_t)(sign | inf);"),
    ("sym_codes_by_reciprocal", "c[j] = sat_rne(v[j] / sc, code_lo, code_hi);",
     "c[j] = sat_rne(v[j] * (1.0f / sc), code_lo, code_hi);"),
    ("asym_codes_by_reciprocal", "float q = v[j] / sc;", "float q = v[j] * (1.0f / sc);"),
    ("asym_qhi_by_reciprocal", "float q_hi = hi / sc;", "float q_hi = hi * (1.0f / sc);"),
    ("sym_scale_by_reciprocal", "float sc = amax / offset_opt;", "float sc = amax * (1.0f / offset_opt);"),
    ("asym_scale_by_reciprocal", "float sc = range / scale_opt;", "float sc = range * (1.0f / scale_opt);"),
    ("asym_offset_one_rounding", "float off = offset_opt - q_hi;",
     "float off = (float)((double)offset_opt - (double)hi / (double)sc);"),
    ("asym_code_one_rounding", "float t = q + off;", "float t = (float)((double)v[j] / (double)sc + (double)off);"),
    ("ada_codes_by_reciprocal", "out[row * H + j] = (int8_t)sat_rne((float)yr[j] / qs, -128, 127);",
     "out[row * H + j] = (int8_t)sat_rne((float)yr[j] * (1.0f / qs), -128, 127);"),
    ("ada_scale_by_reciprocal", "float qs = amax / 127.0f;", "float qs = amax * (1.0f / 127.0f);"),
    ("ada_codes_in_binary64", "out[row * H + j] = (int8_t)sat_rne((float)yr[j] / qs, -128, 127);",
     "out[row * H + j] = (int8_t)sat_rne((float)(yr[j] / (double)qs), -128, 127);"),
    ("aq_distributed_offset", "float u = v + o;\n                t = u * s;",
     "float u = v * s;\n                t = u + o * s;"),
    ("aq_fused_offset", "float u = v + o;\n                t = u * s;",
     "float u = o * s;\n                t = fmaf(v, s, u);"),
    ("aq_binary64_affine", "float u = v + o;\n                t = u * s;",
     "double u = (double)v + o;\n                t = (float)(u * s);"),
    ("mx_amax_signed", "else if (fabs((double)v) > amax)\n                    amax = fabs((double)v);",
     "else if ((double)v > amax)\n                    amax = (double)v;"),
]


def _run_pins(orc):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
            break
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) == 1, f"mutation anchor for {name} must occur exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(text.replace(old, new), encoding="utf-8")
    lib = tmp_path / "libmutant.so"
    oracle.build(str(mutant_src), str(lib))
    failed = _run_pins(oracle.Oracle(str(lib)))
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "copy.c"
    shutil.copy(SRC, src)
    lib = tmp_path / "libcopy.so"
    oracle.build(str(src), str(lib))
    assert _run_pins(oracle.Oracle(str(lib))) == []
