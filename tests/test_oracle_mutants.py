"""CPU-only: the pins catch plausible mistakes planted in a copy of the oracle.

Each mutant is a textual edit of ``oracle/oracle.c`` (a dropped term, a wrong
sign, index or bias), compiled with gcc into a temporary library.  The test
passes when at least one pin fails on it; the shipped oracle is untouched.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.LIB_PATH), "oracle.c")

MUTANTS = {
    "butterfly_sign": ("x[base + j + stride] = a - b;", "x[base + j + stride] = b - a;"),
    "fwht_dropped_stage": ("stride < n; stride <<= 1", "stride < n / 2; stride <<= 1"),
    "fwht_strides_descending": ("for (int64_t stride = 1; stride < n; stride <<= 1) {",
                                "for (int64_t stride = n >> 1; stride >= 1; stride >>= 1) {"),
    "scale_not_sqrt": ("1.0 / sqrt((double)group)", "1.0 / (double)group"),
    "scale_in_fp32": ("    return (float)((double)v * scale);", "    return v * (float)scale;"),
    "index_msb_first": ("idx |= bit << j;", "idx |= bit << (m->bits - 1 - j);"),
    "index_wrong_stride": ("int64_t t = m->bits * col + j;", "int64_t t = 4 * col + j;"),
    "matvec_dropped_norm": ("acc += norm * part;", "acc += part;"),
    "matvec_wrong_norm_index": ("m->norms[row * n_groups + g]);\n            acc",
                                "m->norms[row * n_groups]);\n            acc"),
    "prepare_no_pad_zero": ("p[k] = k < m->input ? x[k] : 0.0f;", "p[k] = k < m->input ? x[k] : 1.0f;"),
    "dequant_dropped_norm": ("tg[k] = m->codebook[oracle_cq_index(m, row, g * m->group + k)] * norm;",
                             "tg[k] = m->codebook[oracle_cq_index(m, row, g * m->group + k)];"),
    "dense_dropped_column": ("for (int64_t c = 0; c < m->input; c++) acc +=",
                             "for (int64_t c = 1; c < m->input; c++) acc +="),
    "dequant_no_transform": ("        oracle_fwht(tg, m->group);\n        for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store",
                             "        for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store"),
    "dequant_no_scale": ("for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store(tg[k], m->group);",
                         "for (int64_t k = 0; k < m->group; k++) tg[k] = tg[k];"),
    "dequant_norm_of_group_0": ("float norm = oracle_f16(m->norms[row * n_groups + g]);",
                                "float norm = oracle_f16(m->norms[row * n_groups]);"),
    "dequant_norm_after_transform": (
        "            tg[k] = m->codebook[oracle_cq_index(m, row, g * m->group + k)] * norm;\n"
        "        oracle_fwht(tg, m->group);\n"
        "        for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store(tg[k], m->group);",
        "            tg[k] = m->codebook[oracle_cq_index(m, row, g * m->group + k)];\n"
        "        oracle_fwht(tg, m->group);\n"
        "        for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store(tg[k] * norm, m->group);"),
    "gather_mag_unscaled": ("gmag[i * m->input + k] = s * inv;", "gmag[i * m->input + k] = s;"),
    "matvec_mag_no_norm": ("amag += fabs(norm) * apart;", "amag += apart;"),
    "matvec_mag_signed": ("apart += fabs(term);", "apart += term;"),
    "f8_mag_signed": ("(double)oracle_e8m0(s[sr * SC + sc]) * (double)x[c];\n            acc += term;\n            amag += fabs(term);",
                      "(double)oracle_e8m0(s[sr * SC + sc]) * (double)x[c];\n            acc += term;\n            amag += term;"),
    "i8_mag_signed": ("(double)oracle_e8m0(s[r * ns + c / G]) *\n                          (double)x[c];\n            acc += term;\n            amag += fabs(term);",
                      "(double)oracle_e8m0(s[r * ns + c / G]) *\n                          (double)x[c];\n            acc += term;\n            amag += term;"),
    "f16_bias": ("ldexp((double)(1024 + F), E - 25)", "ldexp((double)(1024 + F), E - 26)"),
    "f16_subnormal_bias": ("ldexp((double)F, -24)", "ldexp((double)F, -25)"),
    "f16_hidden_bit_dropped": ("ldexp((double)(1024 + F), E - 25)", "ldexp((double)F, E - 25)"),
    "f16_sign_dropped": ("return (float)(negative ? -magnitude : magnitude);", "return (float)magnitude;"),
    "e4m3_subnormal_exp": ("v = ldexp((double)mant / 8.0, 1 - 7);", "v = ldexp((double)mant / 8.0, 0 - 7);"),
    "e4m3_no_clamp": ("if (v > 448.0) v = 448.0;", ""),
    "e4m3_sign_dropped": ("return (float)(s ? -v : v);", "return (float)v;"),
    "e8m0_bias": ("ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 128)"),
    "f8_scale_col_uses_R": ("int64_t sc = (c * SC) / C;", "int64_t sc = (c * SC) / R;"),
    "f8_scale_row_transposed": ("int64_t sr = (r * SR) / R;", "int64_t sr = (r * SC) / R;"),
    "xorshift_wrong_shift": ("s ^= s >> 17;", "s ^= s >> 15;"),
    "topk_ties_by_higher_index": ("return a < b ? -1 : (a > b ? 1 : 0);", "return a < b ? 1 : (a > b ? -1 : 0);"),
    "topk_nan_first": ("if (na != nb) return na ? 1 : -1;", "if (na != nb) return na ? -1 : 1;"),
    "sample_no_temperature": ("exp(((double)vals[i] - (double)vals[0]) / temperature);\n        if",
                              "exp(((double)vals[i] - (double)vals[0]));\n        if"),
    "topk_plus_zero_above_minus_zero": (
        "if (!na && va != vb) return va > vb ? -1 : 1;",
        "if (!na && (va != vb || signbit(va) != signbit(vb)))\n"
        "        return (va > vb || (va == vb && !signbit(va))) ? -1 : 1;"),
    "sample_nan_weighted": ("S += isnan(vals[i]) ? 0.0 : exp(", "S += isnan(vals[i]) ? 1.0 : exp("),
    "sample_greedy_only_on_nan": ("if (temperature <= 0.0 || k == 1 || !isfinite(vals[0])) return ids[0];",
                                  "if (temperature <= 0.0 || k == 1 || isnan(vals[0])) return ids[0];"),
    "sample_top_not_subtracted": (
        "        S += isnan(vals[i]) ? 0.0 : exp(((double)vals[i] - (double)vals[0]) / temperature);\n"
        "    double target = u * S, run = 0.0;\n"
        "    for (int64_t i = 0; i < k; i++) {\n"
        "        run += isnan(vals[i]) ? 0.0 : exp(((double)vals[i] - (double)vals[0]) / temperature);",
        "        S += isnan(vals[i]) ? 0.0 : exp((double)vals[i] / temperature);\n"
        "    double target = u * S, run = 0.0;\n"
        "    for (int64_t i = 0; i < k; i++) {\n"
        "        run += isnan(vals[i]) ? 0.0 : exp((double)vals[i] / temperature);"),
    "sample_cdf_off_by_one": ("if (target < run) return ids[i];", "if (target <= run) return ids[i > 0 ? i - 1 : 0];"),
    "sample_u_over_2_32_minus_1": ("(double)*state / 4294967296.0", "(double)*state / 4294967295.0"),
    "i8_group_fixed_16": ("(double)oracle_e8m0(s[r * ns + c / G])", "(double)oracle_e8m0(s[r * ns + c / 16])"),
    "i8_scale_dropped": ("double term = (double)w[r * C + c] * (double)oracle_e8m0(s[r * ns + c / G]) *",
                         "double term = (double)w[r * C + c] * 1.0 *"),
    "int8_ties_away": ("q[i] = js_to_int8(nearbyint((double)v[i] / scale));",
                       "q[i] = js_to_int8(round((double)v[i] / scale));"),
    "int8_signed_max": ("maximum = js_max(maximum, fabs((double)v[i]));", "maximum = js_max(maximum, (double)v[i]);"),
    "int8_scale_128": ("double scale = maximum / 127.0;", "double scale = maximum / 128.0;"),
    "int8_divides_by_fp32_scale": ("double scale = maximum / 127.0;",
                                   "double scale = (double)(float)(maximum / 127.0);"),
    "int8_no_floor": ("double maximum = 1e-12;", "double maximum = 0.0;"),
    "int8_dot_scale_dropped": ("if (y) y[i] = (double)scales[r] * acc;", "if (y) y[i] = acc;"),
    "dense_sum_in_fp32": ("        double acc = 0.0;\n        for (int64_t c = 0; c < m->input; c++) acc +=",
                          "        float acc = 0.0f;\n        for (int64_t c = 0; c < m->input; c++) acc +="),
    "gather_scale_in_fp32": (
        "for (int64_t k = 0; k < m->group; k++) tg[k] = scale_store(tg[k], m->group);\n    }\n    memcpy",
        "for (int64_t k = 0; k < m->group; k++) tg[k] = tg[k] * (float)(1.0 / sqrt((double)m->group));\n    }\n    memcpy"),
    "hmlp_silu_in_fp32": ("z[i] = (float)(t / (1.0 + exp(-t)));", "z[i] = (float)t / (1.0f + expf(-(float)t));"),
    "hmlp_scale_in_fp32": ("for (int64_t i = 0; i < H; i++) z[i] = (float)((double)z[i] * scale);",
                           "for (int64_t i = 0; i < H; i++) z[i] = z[i] * (float)scale;"),
    "hmlp_update_one_rounding": ("out[i] = u ? (float)((double)block - (double)u[i]) : block;",
                                 "out[i] = u ? (float)((double)resid[i] + (double)z[i] - (double)u[i]) : block;"),
    "hmlp_silu_sign": ("z[i] = (float)(t / (1.0 + exp(-t)));", "z[i] = (float)(t / (1.0 + exp(t)));"),
    "hmlp_pad_ones": ("z[i] = i < hidden ? n[i] : 0.0f;", "z[i] = i < hidden ? n[i] : 1.0f;"),
    "hmlp_no_d3": ("z[i] = (float)((double)z[i] * (double)d3[i]);", ""),
    "hmlp_unnormalized": ("double scale = 1.0 / sqrt((double)H);", "double scale = 1.0;"),
    "hmlp_mag_l1_unscaled": ("fabs((double)d3[i]) / sqrt((double)H) * l1;", "fabs((double)d3[i]) * l1;"),
    "hmlp_u_added": ("out[i] = u ? (float)((double)block - (double)u[i]) : block;",
                     "out[i] = u ? (float)((double)block + (double)u[i]) : block;"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique or missing"
    mutated = tmp_path / f"{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    inc = os.path.dirname(SRC)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-I", inc, "-o", str(lib), str(mutated), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    oracle.use_library(lib)
    try:
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
                break
        assert caught, f"no pin fails on mutant {name}"
    finally:
        oracle.use_library(None)
