"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutation below is a plausible slip (a wrong sign, index, stride or
constant, a dropped term, a swapped order, a wrong rounding rule) applied to
the first occurrence of a line of ``oracle/convrot_oracle.c``.  The mutated
copy is compiled with the oracle's own flags into a temporary directory; the
real oracle is never modified.  All mutations keep every access in bounds.
"""
import subprocess

import pytest

import oracle
import pins

MUTATIONS = {
    "butterfly_sign": ("g[i] = h - x3;", "g[i] = h + x3;"),
    "butterfly_index": ("g[i + st] = h - x2;", "g[i + st] = h - x1;"),
    "butterfly_sum_term": ("float s = (x0 + x1) + (x2 + x3);", "float s = (x0 + x1) + (x2 - x3);"),
    "butterfly_no_normalization": ("float h = s * 0.5f;", "float h = s;"),
    "stage_stride": ("for (int st = 1; st < G; st *= 4)\n        h4_stage_f32",
                     "for (int st = 1; st < G; st *= 16)\n        h4_stage_f32"),
    "stage_skipped": ("for (int st = 1; st < G; st *= 4)\n        h4_stage_f32",
                      "for (int st = 4; st < G; st *= 4)\n        h4_stage_f32"),
    "f64_butterfly_sign": ("g[i + 3 * st] = h - x0;\n    }\n}\n\nstatic void rotate_group_f64",
                           "g[i + 3 * st] = h + x0;\n    }\n}\n\nstatic void rotate_group_f64"),
    "scale_constant": ("*s_out = m / 127.0f;", "*s_out = m / 128.0f;"),
    "inverse_constant": ("float inv = 127.0f / m;", "float inv = 128.0f / m;"),
    "round_truncate": ("float t = rintf(y[i] * inv);", "float t = truncf(y[i] * inv);"),
    "round_half_away": ("float t = rintf(y[i] * inv);", "float t = roundf(y[i] * inv);"),
    "per_group_max": ("for (int64_t i = 0; i < K; ++i) {\n        float a = fabsf(y[i]);",
                      "for (int64_t i = 0; i < G; ++i) {\n        float a = fabsf(y[i]);"),
    "prescale_divides": ("y[i] = y[i] * alpha;", "y[i] = y[i] / alpha;"),
    "unscale_multiplies": ("t = t / alpha;", "t = t * alpha;"),
    "unscale_after_bias": ("            if (alpha != 1.0f)\n                t = t / alpha;\n"
                           "            if (bias)\n                t = t + bias[o];",
                           "            if (bias)\n                t = t + bias[o];\n"
                           "            if (alpha != 1.0f)\n                t = t / alpha;"),
    "scale_order_swapped": ("            t = t * s_x[r];\n            if (s_w)\n                t = t * s_w[o];",
                            "            if (s_w)\n                t = t * s_w[o];\n            t = t * s_x[r];"),
    "gemm_reversed_index": ("acc += (int64_t)Qx[r * K + i] * (int64_t)Qw[o * K + i];",
                            "acc += (int64_t)Qx[r * K + (K - 1 - i)] * (int64_t)Qw[o * K + i];"),
    "gemm_dropped_term": ("for (int64_t i = 0; i < K; ++i)\n                acc +=",
                          "for (int64_t i = 1; i < K; ++i)\n                acc +="),
    "pack_tail_offset": ("uint8_t *tail = packed + m_pad * K;", "uint8_t *tail = packed + M * K;"),
    "pad_rows_unwritten": ("            else\n                memset(Q + r * K, 0, (size_t)K);\n", "\n"),
    "bf16_widen": ("uint32_t u = (uint32_t)((const uint16_t *)X)[idx] << 16;",
                   "uint32_t u = (uint32_t)((const uint16_t *)X)[idx] << 15;"),
    "bf16_round_half_up": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    "modulate_folded": ("const float xs = x * scale[i];\n            float y = x + xs;",
                        "const float xs = 1.0f + scale[i];\n            float y = x * xs;"),
    "modulate_shift_first": ("float y = x + xs;\n            if (shift)\n                y = y + shift[i];",
                             "float y = x;\n            if (shift)\n                y = y + shift[i];\n            y = y + xs;"),
    "modulate_scale_index": ("const float xs = x * scale[i];", "const float xs = x * scale[K - 1 - i];"),
    "int4_high_nibble_first": ("const int nib = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
                               "const int nib = (k % 2 == 0) ? (byte >> 4) : (byte & 0x0F);"),
    "int4_offset_binary": ("Qw[o * K + k] = (int8_t)(nib >= 8 ? nib - 16 : nib);",
                           "Qw[o * K + k] = (int8_t)(nib - 8);"),
    "residual_before_gate": ("            t = t * gate[o];\n            t = t + load_widened(R, r_dtype, r * ldr + o);",
                             "            t = t + load_widened(R, r_dtype, r * ldr + o);\n            t = t * gate[o];"),
    "gate_scale_fused": ("            if (scale != 1.0f)\n                t = t * scale;\n            t = t * gate[o];",
                         "            t = t * (scale * gate[o]);"),
    "gate_row_index": ("t = t * gate[o];", "t = t * gate[r % N];"),
    "zero_row_scale": ("        *s_out = 0.0f;\n        memset(q, 0, (size_t)K);\n        return;",
                       "        m = 1.0f;"),
    "rms_sum_not_mean": ("const float mean = S / (float)K;", "const float mean = S;"),
    "rms_eps_after_root": ("const float d = sqrtf(mean + eps);", "const float d = sqrtf(mean) + eps;"),
    "rms_no_reciprocal": ("const float rs = 1.0f / d;", "const float rs = d;"),
    "rms_abs_not_square": ("sq[i] = x * x;", "sq[i] = fabsf(x);"),
    "rms_weight_reversed": ("y = y * weight[i];", "y = y * weight[K - 1 - i];"),
    "rms_last_block_only": ("S = b == 0 ? block : S + block;", "S = block;"),
    "norm_var_uncentered": ("const float dv = load_widened(X, x_dtype, r * ldx + b + i) - mean;",
                            "const float dv = load_widened(X, x_dtype, r * ldx + b + i);"),
    "norm_output_uncentered": ("const float dv = load_widened(X, x_dtype, r * ldx + i) - mean;",
                               "const float dv = load_widened(X, x_dtype, r * ldx + i);"),
    "norm_var_sum_not_mean": ("const float var = S2 / (float)K;", "const float var = S2;"),
    "norm_mean_over_blocks": ("const float mean = S1 / (float)K;", "const float mean = S1 / (float)(K / 64);"),
    "norm_eps_after_root": ("const float sd = sqrtf(var + eps);", "const float sd = sqrtf(var) + eps;"),
    "norm_no_reciprocal": ("const float rs = 1.0f / sd;", "const float rs = sd;"),
    "norm_weight_reversed": ("float y = dv * rs;\n            if (weight)\n                y = y * weight[i];",
                             "float y = dv * rs;\n            if (weight)\n                y = y * weight[K - 1 - i];"),
    "norm_last_block_only": ("S2 = b == 0 ? block : S2 + block;", "S2 = block;"),
    "act_exp_sign": ("const float e = oracle_expf(-g);", "const float e = oracle_expf(g);"),
    "act_no_one": ("const float d = 1.0f + e;", "const float d = e;"),
    "act_silu_is_sigmoid": ("const float a = act == ORACLE_ACT_SILU ? g * sg : sg;", "const float a = sg;"),
    "act_no_up": ("Y[r * K + i] = a * u;", "Y[r * K + i] = a;"),
    "act_exp_binary32_series": ("return (float)expl((long double)x);",
                                "return 1.0f + x * (1.0f + x * (0.5f + x * (1.0f / 6.0f)));"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    c.write_text(mutated)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(c), "-o", str(so), "-lm"], check=True,
                   capture_output=True)
    return oracle.Oracle(str(so))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    mutant = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError) as e:
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
