"""Plant one plausible mistake at a time in a copy of the CPU oracle and check
that the pins catch every one.  The copies are built in a temporary folder;
the real oracle source is never modified."""
import os
import re
import subprocess

import pytest

import oracle
from tests import pins

# (name, function of ds_sel_oracle.c, text in that function, replacement)
MUTANTS = [
    ("drop_last_head", "score_fp32", "for (int h = 0; h < heads; ++h) {",
     "for (int h = 0; h < heads - 1; ++h) {"),
    ("drop_last_dim", "score_fp32", "for (int i = 0; i < dim; ++i) {", "for (int i = 0; i < dim - 1; ++i) {"),
    ("ignore_head_weight", "score_fp32", "float t = bf16_bits_to_float(w_row[h]) * dot;", "float t = dot;"),
    ("head_index_reversed", "score_fp32", "const uint16_t* qh = q_row + (int64_t)h * dim;",
     "const uint16_t* qh = q_row + (int64_t)(heads - 1 - h) * dim;"),
    ("sign_flip", "score_fp32", "s = s + t;", "s = s - t;"),
    ("tie_to_higher_index", "by_score_desc_then_index", "if (a->block < b->block) return -1;",
     "if (a->block < b->block) return 1;"),
    ("ascending_order", "by_score_desc_then_index", "if (a->score > b->score) return -1;",
     "if (a->score > b->score) return 1;"),
    ("limit_drops_last", "ds_sel_oracle_select", "for (int64_t b = 0; b < lim; ++b) {",
     "for (int64_t b = 0; b + 1 < lim; ++b) {"),
    ("mask_bit_order_reversed", "mask_bit", "(uint32_t)(b & 31)", "(uint32_t)(31 - (b & 31))"),
    ("mask_ignored", "ds_sel_oracle_select", "if (mrow && !mask_bit(mrow, b)) continue;", ""),
    ("no_limit_clamp_low", "clamped_limit", "if (v < 0) v = 0;", "if (v < 0) v = -v;"),
    ("padding_score_zero", "ds_sel_oracle_select", "os[j] = -INFINITY;", "os[j] = 0.0f;"),
    ("count_is_admitted", "ds_sel_oracle_select", "if (out_count) out_count[lr] = (int32_t)m;",
     "if (out_count) out_count[lr] = (int32_t)n;"),
    ("wrong_row_of_w", "ds_sel_oracle_select", "const uint16_t* w_row = w + lr * heads;",
     "const uint16_t* w_row = w + (int64_t)l * rows * heads;"),
    ("shared_mask_ignores_row", "ds_sel_oracle_select", "mask + l * mask_layer_stride + r * mask_row_stride",
     "mask + l * mask_layer_stride"),
    ("score_blocks_no_layer_stride", "ds_sel_oracle_score_blocks",
     "keys + layer * key_layer_stride + (int64_t)list[j] * ldk", "keys + (int64_t)list[j] * ldk"),
    ("score_blocks_row_offset", "ds_sel_oracle_score_blocks", "int64_t lr = (int64_t)layer * rows + row;",
     "int64_t lr = (int64_t)row;"),
    ("score_blocks_layer_as_row", "ds_sel_oracle_score_blocks", "int64_t lr = (int64_t)layer * rows + row;",
     "int64_t lr = (int64_t)row * rows + layer;"),
    # the per-head ReLU score
    ("relu_dropped", "score_relu_fp32", "float r = dot > 0.0f ? dot : 0.0f;", "float r = dot;"),
    ("relu_inverted", "score_relu_fp32", "float r = dot > 0.0f ? dot : 0.0f;",
     "float r = dot < 0.0f ? dot : 0.0f;"),
    ("relu_after_weight", "score_relu_fp32", "float t = bf16_bits_to_float(w_row[h]) * r;",
     "float t = bf16_bits_to_float(w_row[h]) * dot; t = t > 0.0f ? t : 0.0f;"),
    ("relu_also_on_the_sum", "score_relu_fp32", "return s + 0.0f;", "return (s > 0.0f ? s : 0.0f) + 0.0f;"),
    ("relu_head_index_reversed", "score_relu_fp32", "const uint16_t* qh = q_row + (int64_t)h * dim;",
     "const uint16_t* qh = q_row + (int64_t)(heads - 1 - h) * dim;"),
    ("relu_drop_last_dim", "score_relu_fp32", "for (int i = 0; i < dim; ++i) {",
     "for (int i = 0; i < dim - 1; ++i) {"),
    ("relu_sign_flip", "score_relu_fp32", "s = s + t;", "s = s - t;"),
    ("relu_limit_drops_last", "ds_sel_oracle_select_relu", "for (int64_t b = 0; b < lim; ++b) {",
     "for (int64_t b = 0; b + 1 < lim; ++b) {"),
    ("relu_mask_ignored", "ds_sel_oracle_select_relu", "if (mrow && !mask_bit(mrow, b)) continue;", ""),
    ("relu_padding_score_zero", "ds_sel_oracle_select_relu", "os[j] = j < m ? list[j].score : -INFINITY;",
     "os[j] = j < m ? list[j].score : 0.0f;"),
    ("relu_count_is_admitted", "ds_sel_oracle_select_relu", "if (out_count) out_count[lr] = (int32_t)m;",
     "if (out_count) out_count[lr] = (int32_t)n;"),
    ("relu_wrong_row_of_w", "ds_sel_oracle_select_relu", "const uint16_t* w_row = w + lr * heads;",
     "const uint16_t* w_row = w + (int64_t)l * rows * heads;"),
    ("relu_score_blocks_row_offset", "ds_sel_oracle_score_blocks_relu",
     "int64_t lr = (int64_t)layer * rows + row;", "int64_t lr = (int64_t)row;"),
    # the 8-bit key stream
    ("q8_scale_not_divided", "ds_sel_oracle_quantize_q8", "float_to_half_bits(amax / 127.0f)",
     "float_to_half_bits(amax)"),
    ("q8_codes_truncated", "ds_sel_oracle_quantize_q8", "float r = roundf(bf16_bits_to_float(x[32 * g + i]) / s);",
     "float r = truncf(bf16_bits_to_float(x[32 * g + i]) / s);"),
    ("q8_ties_to_even", "ds_sel_oracle_quantize_q8", "float r = roundf(bf16_bits_to_float(x[32 * g + i]) / s);",
     "float r = rintf(bf16_bits_to_float(x[32 * g + i]) / s);"),
    ("q8_half_rounding_truncates", "float_to_half_bits",
     "if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;", ""),
    ("q8_half_exponent_off", "half_bits_to_float", "u = sign | ((exp + 112u) << 23) | (man << 13);",
     "u = sign | ((exp + 111u) << 23) | (man << 13);"),
    ("q8_group_of_16", "score_q8_fp32", "float k = half_bits_to_float(scale[i / 32]) * (float)code[i];",
     "float k = half_bits_to_float(scale[i / 16]) * (float)code[i];"),
    ("q8_scale_ignored", "score_q8_fp32", "float k = half_bits_to_float(scale[i / 32]) * (float)code[i];",
     "float k = (float)code[i];"),
    ("q8_scale_layer_dropped", "ds_sel_oracle_select_q8", "scales + l * scale_layer_stride + b * lds, heads, dim);",
     "scales + b * lds, heads, dim);"),
    ("q8_drop_last_head", "score_q8_fp32", "for (int h = 0; h < heads; ++h) {",
     "for (int h = 0; h < heads - 1; ++h) {"),
    ("q8_drop_last_dim", "score_q8_fp32", "for (int i = 0; i < dim; ++i) {", "for (int i = 0; i < dim - 1; ++i) {"),
    ("q8_ignore_head_weight", "score_q8_fp32", "float t = bf16_bits_to_float(w_row[h]) * dot;", "float t = dot;"),
    ("q8_sign_flip", "score_q8_fp32", "s = s + t;", "s = s - t;"),
    ("q8_head_index_reversed", "score_q8_fp32", "const uint16_t* qh = q_row + (int64_t)h * dim;",
     "const uint16_t* qh = q_row + (int64_t)(heads - 1 - h) * dim;"),
    ("q8_limit_drops_last", "ds_sel_oracle_select_q8", "for (int64_t b = 0; b < lim; ++b) {",
     "for (int64_t b = 0; b + 1 < lim; ++b) {"),
    ("q8_mask_ignored", "ds_sel_oracle_select_q8", "if (mrow && !mask_bit(mrow, b)) continue;", ""),
    ("q8_padding_score_zero", "ds_sel_oracle_select_q8", "os[j] = -INFINITY;", "os[j] = 0.0f;"),
    ("q8_count_is_admitted", "ds_sel_oracle_select_q8", "if (out_count) out_count[lr] = (int32_t)m;",
     "if (out_count) out_count[lr] = (int32_t)n;"),
    ("q8_wrong_row_of_w", "ds_sel_oracle_select_q8", "const uint16_t* w_row = w + lr * heads;",
     "const uint16_t* w_row = w + (int64_t)l * rows * heads;"),
    # attention over the selection
    ("attend_no_max_shift", "ds_sel_oracle_attend", "const double p = exp(s[j] - smax);",
     "const double p = exp(s[j]);"),
    ("attend_value_of_slot", "ds_sel_oracle_attend", "V + (int64_t)sel[j] * ldv", "V + (int64_t)j * ldv"),
    ("attend_key_of_slot", "ds_sel_oracle_attend", "K + (int64_t)sel[j] * ldk", "K + (int64_t)j * ldk"),
    ("attend_no_scale", "ds_sel_oracle_attend", "s[j] = scale * dot;", "s[j] = dot;"),
    ("attend_divide_by_count", "ds_sel_oracle_attend", "oh[i] /= z;", "oh[i] /= c;"),
]


def function_span(src, name):
    """[start, end) of the definition of function `name` in the oracle source:
    from its signature to the closing brace of its body."""
    m = re.search(r"^[A-Za-z_][\w \*]*?\b" + re.escape(name) + r"\(", src, re.M)
    assert m, f"no function {name}"
    depth, i = 0, src.index("{", m.end())
    for j in range(i, len(src)):
        depth += {"{": 1, "}": -1}.get(src[j], 0)
        if depth == 0:
            return m.start(), j + 1
    raise AssertionError(f"unbalanced braces in {name}")


@pytest.mark.parametrize("name,func,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, func, old, new):
    with open(oracle.SOURCE) as f:
        src = f.read()
    a, b = function_span(src, func)
    assert old in src[a:b], f"mutation site for {name} is not in {func}"
    mutated = src[:a] + src[a:b].replace(old, new, 1) + src[b:]
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(mutated)
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(output=lib_path, source=str(mutant_src))
    lib = oracle.load(lib_path)
    with pytest.raises((AssertionError, oracle.OracleError)):
        pins.all_pins(lib)


def test_unmutated_copy_passes(tmp_path):
    lib_path = str(tmp_path / "libcopy.so")
    oracle.build(output=lib_path)
    pins.all_pins(oracle.load(lib_path))
