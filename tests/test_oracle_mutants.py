"""Planted mistakes in the oracle (CPU only): every mutant must fail some pin.

Each mutant is oracle.c with one plausible slip written in (a dropped term, a
wrong sign or index, a transposed operand, a format error), compiled with gcc
into a temporary library.  The real oracle passes every pin
(tests/test_oracle_pins.py); a mutant that passed them all would show a gap in
the pins.
"""
from pathlib import Path

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "query_transposed": ("oracle_bf16_value(qh[d])",
                         "oracle_bf16_value(q_bits[((int64_t)b * HD + d) * NH + h])"),
    "last_head_dropped": ("for (int h = 0; h < NH; ++h)", "for (int h = 0; h < NH - 1; ++h)"),
    "last_dim_dropped": ("for (int d = 0; d < HD; ++d) dot +=", "for (int d = 0; d < HD - 1; ++d) dot +="),
    "relu_after_weight": ("acc += (double)weights[(int64_t)b * NH + h] * relu(s * dot);",
                          "acc += relu((double)weights[(int64_t)b * NH + h] * s * dot);"),
    "scale_after_relu": ("relu(s * dot)", "s * relu(dot)"),
    "no_relu": ("(x > 0.0 ? x : 0.0)", "(x)"),
    "relu_drops_nan": ("isnan(x) ? x : (x > 0.0 ? x : 0.0)", "(x > 0.0 ? x : 0.0)"),
    "page_table_ignored": ("const int32_t g = table_ok ? page_table[tr * pt_stride + j] : -1;",
                           "const int32_t g = table_ok ? j : -1;"),
    "table_row_stride_ignored": ("page_table[tr * pt_stride + j]", "page_table[j]"),
    "mask_off_by_one": ("if (p >= L) { o[i] = -INFINITY; continue; }",
                        "if (p > L) { o[i] = -INFINITY; continue; }"),
    "e4m3_bias_8": ("(int)e - 7", "(int)e - 8"),
    "e4m3_subnormal_exp": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "e4m3_sign_lost": ("return s ? -mag : mag;", "return mag;"),
    "e4m3_no_nan": ("if (e == 15u && m == 7u) return NAN;", ""),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "key_slot_uses_page_index": ("(int64_t)g * kv_stride + (int64_t)i * HD;",
                                 "(int64_t)g * kv_stride + (int64_t)j * HD;"),
    "scale_slot_ignored": ("ks + (int64_t)g * ks_stride + 4 * i", "ks + (int64_t)g * ks_stride"),
    "weights_ignore_row": ("weights[(int64_t)b * NH + h]", "weights[h]"),
    "bad_page_not_nan": ("if (!page_ok) { o[i] = NAN; continue; }",
                         "if (!page_ok) { o[i] = 0.0; continue; }"),
    "bf16_keys_scaled": ("        s = 1.0;\n", "        s = 0.5;\n"),
    "encode_ties_up": ("(d == best_d && (c & 1u) == 0u)", "(d == best_d)"),
    "encode_zero_unsigned": ("return signbit(y) ? (best | 0x80u) : best;",
                             "return y < 0.0f ? (best | 0x80u) : best;"),
    "quant_scale_447": ("amax / 448.0f", "amax / 447.0f"),
    "quant_amax_signed": ("const float m = fabsf(k[d]);", "const float m = k[d];"),
    "quant_last_dim_dropped": ("for (int d = 0; d < HD; ++d) {\n      const uint32_t u",
                               "for (int d = 0; d < HD - 1; ++d) {\n      const uint32_t u"),
    "quant_zero_scale": ("amax > 0.0f ? amax / 448.0f : 1.0f", "amax / 448.0f"),
    "request_map_ignored": ("const int64_t tr = row_table ? (int64_t)row_table[b] : (int64_t)b;",
                            "const int64_t tr = (int64_t)b;"),
    "request_map_unchecked": ("const int table_ok = row_table == NULL || (tr >= 0 && tr < num_tables);",
                              "const int table_ok = row_table == NULL || tr >= 0;"),
    "topk_ties_to_high_position": ("return (x->p > y->p) - (x->p < y->p);",
                                   "return (x->p < y->p) - (x->p > y->p);"),
    "topk_nan_first": ("if (xn != yn) return xn - yn;", "if (xn != yn) return yn - xn;"),
    "topk_smallest": ("return x->v > y->v ? -1 : 1;", "return x->v < y->v ? -1 : 1;"),
    "topk_ignores_length": ("    int32_t L = seqlens[b];\n    if (L < 0) L = 0;\n    if (L > ncols) L = ncols;\n    const int32_t m",
                            "    int32_t L = ncols;\n    const int32_t m"),
    "topk_rank_order_output": ("      qsort(o, (size_t)m, sizeof(int32_t), topk_pos_cmp);\n", ""),
    "topk_signed_zero_ordered": (
        "  if (!xn && x->v != y->v) return x->v > y->v ? -1 : 1;\n",
        "  if (!xn && x->v != y->v) return x->v > y->v ? -1 : 1;\n"
        "  if (!xn && signbit(x->v) != signbit(y->v)) return signbit(x->v) ? 1 : -1;\n"),
    "topk_pad_zero": ("for (int32_t t = m; t < k; ++t) o[t] = -1;",
                      "for (int32_t t = m; t < k; ++t) o[t] = 0;"),
}


@pytest.fixture(scope="module")
def source():
    return oracle.SOURCE.read_text()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path: Path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib = oracle.build(src, tmp_path / f"liboracle_{name}.so")
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
