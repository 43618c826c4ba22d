"""Plant one plausible mistake at a time in a copy of the CPU oracle and check
that the pins catch every one.  The copies are built in a temporary folder;
the real oracle source is never modified."""
import os
import subprocess

import pytest

import oracle
from tests import pins

# (name, text in ds_sel_oracle.c, replacement)
MUTANTS = [
    ("drop_last_head", "for (int h = 0; h < heads; ++h) {", "for (int h = 0; h < heads - 1; ++h) {"),
    ("drop_last_dim", "for (int i = 0; i < dim; ++i) {", "for (int i = 0; i < dim - 1; ++i) {"),
    ("ignore_head_weight", "float t = bf16_bits_to_float(w_row[h]) * dot;", "float t = dot;"),
    ("head_index_reversed", "const uint16_t* qh = q_row + (int64_t)h * dim;",
     "const uint16_t* qh = q_row + (int64_t)(heads - 1 - h) * dim;"),
    ("sign_flip", "s = s + t;", "s = s - t;"),
    ("tie_to_higher_index", "if (a->block < b->block) return -1;", "if (a->block < b->block) return 1;"),
    ("ascending_order", "if (a->score > b->score) return -1;", "if (a->score > b->score) return 1;"),
    ("limit_drops_last", "for (int64_t b = 0; b < lim; ++b) {", "for (int64_t b = 0; b + 1 < lim; ++b) {"),
    ("mask_bit_order_reversed", "(uint32_t)(b & 31)", "(uint32_t)(31 - (b & 31))"),
    ("mask_ignored", "if (mrow && !mask_bit(mrow, b)) continue;", ""),
    ("no_limit_clamp_low", "if (v < 0) v = 0;", "if (v < 0) v = -v;"),
    ("padding_score_zero", "os[j] = -INFINITY;", "os[j] = 0.0f;"),
    ("count_is_admitted", "if (out_count) out_count[lr] = (int32_t)m;",
     "if (out_count) out_count[lr] = (int32_t)n;"),
    ("wrong_row_of_w", "const uint16_t* w_row = w + lr * heads;", "const uint16_t* w_row = w + (int64_t)l * rows * heads;"),
    ("shared_mask_ignores_row", "mask + l * mask_layer_stride + r * mask_row_stride",
     "mask + l * mask_layer_stride"),
    ("score_blocks_no_layer_stride", "keys + layer * key_layer_stride + (int64_t)list[j] * ldk",
     "keys + (int64_t)list[j] * ldk"),
    ("score_blocks_row_offset", "int64_t lr = (int64_t)layer * rows + row;",
     "int64_t lr = (int64_t)row;"),
    ("score_blocks_layer_as_row", "int64_t lr = (int64_t)layer * rows + row;",
     "int64_t lr = (int64_t)row * rows + layer;"),
    ("q8_scale_not_divided", "float_to_half_bits(amax / 127.0f)", "float_to_half_bits(amax)"),
    ("q8_codes_truncated", "float r = roundf(bf16_bits_to_float(x[32 * g + i]) / s);",
     "float r = truncf(bf16_bits_to_float(x[32 * g + i]) / s);"),
    ("q8_ties_to_even", "float r = roundf(bf16_bits_to_float(x[32 * g + i]) / s);",
     "float r = rintf(bf16_bits_to_float(x[32 * g + i]) / s);"),
    ("q8_half_rounding_truncates", "if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;", ""),
    ("q8_half_exponent_off", "u = sign | ((exp + 112u) << 23) | (man << 13);",
     "u = sign | ((exp + 111u) << 23) | (man << 13);"),
    ("q8_group_of_16", "float k = half_bits_to_float(scale[i / 32]) * (float)code[i];",
     "float k = half_bits_to_float(scale[i / 16]) * (float)code[i];"),
    ("q8_scale_ignored", "float k = half_bits_to_float(scale[i / 32]) * (float)code[i];",
     "float k = (float)code[i];"),
    ("q8_scale_layer_dropped", "scales + l * scale_layer_stride + b * lds, heads, dim);",
     "scales + b * lds, heads, dim);"),
    ("attend_no_max_shift", "const double p = exp(s[j] - smax);", "const double p = exp(s[j]);"),
    ("attend_value_of_slot", "V + (int64_t)sel[j] * ldv", "V + (int64_t)j * ldv"),
    ("attend_key_of_slot", "K + (int64_t)sel[j] * ldk", "K + (int64_t)j * ldk"),
    ("attend_no_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("attend_divide_by_count", "oh[i] /= z;", "oh[i] /= c;"),
]


# The same statements in the 8-bit score loop (second occurrence of each).
MUTANTS += [
    ("q8_drop_last_head", "for (int h = 0; h < heads; ++h) {", "for (int h = 0; h < heads - 1; ++h) {", 2),
    ("q8_drop_last_dim", "for (int i = 0; i < dim; ++i) {", "for (int i = 0; i < dim - 1; ++i) {", 2),
    ("q8_ignore_head_weight", "float t = bf16_bits_to_float(w_row[h]) * dot;", "float t = dot;", 2),
    ("q8_sign_flip", "s = s + t;", "s = s - t;", 2),
    ("q8_head_index_reversed", "const uint16_t* qh = q_row + (int64_t)h * dim;",
     "const uint16_t* qh = q_row + (int64_t)(heads - 1 - h) * dim;", 2),
    ("q8_limit_drops_last", "for (int64_t b = 0; b < lim; ++b) {", "for (int64_t b = 0; b + 1 < lim; ++b) {", 2),
    ("q8_mask_ignored", "if (mrow && !mask_bit(mrow, b)) continue;", "", 2),
    ("q8_padding_score_zero", "os[j] = -INFINITY;", "os[j] = 0.0f;", 2),
    ("q8_count_is_admitted", "if (out_count) out_count[lr] = (int32_t)m;",
     "if (out_count) out_count[lr] = (int32_t)n;", 2),
    ("q8_wrong_row_of_w", "const uint16_t* w_row = w + lr * heads;",
     "const uint16_t* w_row = w + (int64_t)l * rows * heads;", 2),
]


def _site(m):
    """(name, old, new, occurrence): the occurrence of the site that is changed,
    counting from 1; a mutant without one changes the first (the bf16 path
    comes before the 8-bit one in the source)."""
    return m if len(m) == 4 else (*m, 1)


@pytest.mark.parametrize("name,old,new,occurrence", [_site(m) for m in MUTANTS], ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, occurrence):
    with open(oracle.SOURCE) as f:
        src = f.read()
    parts = src.split(old)
    assert len(parts) > occurrence, f"mutation site for {name} has no occurrence {occurrence}"
    mutated = old.join(parts[:occurrence]) + new + old.join(parts[occurrence:])
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
