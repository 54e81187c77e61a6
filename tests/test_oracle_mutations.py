"""Each plausible mistake planted in a copy of the oracle is caught by at least one pin.

The copies are compiled into a temporary directory on the CPU; the oracle itself is not
touched. A mutation that no pin catches would mean the pins leave that part unchecked.
"""
import os

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "diagonal_dropped": ("return !invalid && row >= col;", "return !invalid && row > col;"),
    "length_off_by_one": ("int invalid = row >= L || col >= L;",
                          "int invalid = row > L || col > L;"),
    "upper_triangle": ("return !invalid && row >= col;", "return !invalid && row <= col;"),
    "scale_dropped_in_denominator": ("den += exp(scale * load_elem(x, c, dtype) - mu);",
                                     "den += exp(load_elem(x, c, dtype) - mu);"),
    "sign_flipped_in_numerator": ("y[c] = exp(scale * load_elem(x, c, dtype) - mu) / den;",
                                  "y[c] = exp(mu - scale * load_elem(x, c, dtype)) / den;"),
    "batch_plane_transposed": ("int64_t off = ((b * M + m) * S + r) * S;",
                               "int64_t off = ((m * B + b) * S + r) * S;"),
    "truncating_rounding": ("double q = nearbyint(ldexp(a, pbits - E));",
                            "double q = floor(ldexp(a, pbits - E));"),
    "subnormal_spacing": ("if (E < emin) E = emin;", ""),
    "subnormal_decode": ("mag = ldexp((double)f, 1 - bias - pbits);",
                         "mag = ldexp((double)f, -bias - pbits);"),
    "backward_sign": ("(load_elem(dy, off + c, dtype) - dot);",
                      "(load_elem(dy, off + c, dtype) + dot);"),
    "backward_scale_dropped": ("dx[c] = scale * load_elem(y, off + c, dtype) *",
                               "dx[c] = load_elem(y, off + c, dtype) *"),
    "backward_dot_unmasked": ("if (kept(r, c, L)) dot += load_elem(dy", "dot += load_elem(dy"),
    "backward_rows_row_ignored": ("backward_row(y_rows, dy_rows, i * S, row[i],",
                                  "backward_row(y_rows, dy_rows, i * S, S - 1,"),
    "row_column_swapped": ("if (kept(r, c, L))\n            y[c]",
                           "if (kept(c, r, L))\n            y[c]"),
    # mask variants
    "band_upper_edge_strict": ("return c - r >= lo && c - r <= hi;",
                               "return c - r >= lo && c - r < hi;"),
    "band_lower_edge_ignored": ("return c - r >= lo && c - r <= hi;", "return c - r <= hi;"),
    "band_column_length_ignored": ("if (r >= L || c >= L) return 0;", "if (r >= L) return 0;"),
    "variant_lengths_ignored": ("int64_t L = seq_lens ? valid_length(seq_lens[b], S) : S;",
                                "int64_t L = S;"),
    "mask_inverted": ("mask[b * sb + m * sm + r * sr + c] != 0",
                      "mask[b * sb + m * sm + r * sr + c] == 0"),
    "mask_row_stride_dropped": ("mask[b * sb + m * sm + r * sr + c]", "mask[b * sb + m * sm + c]"),
    "mask_batch_ignored": ("mask[b * sb + m * sm + r * sr + c]", "mask[m * sm + r * sr + c]"),
    "empty_variant_row_uniform": ("    if (nkept == 0) {\n        for (int64_t c = 0; c < S; ++c) y[c] = 0.0;",
                                  "    if (nkept == 0) {\n        for (int64_t c = 0; c < S; ++c) y[c] = 1.0 / (double)S;"),
    "variant_scale_dropped_in_max": ("        double z = scale * load_elem(x, c, dtype);\n        if (z > mu) mu = z;\n        ++nkept;\n    }\n    if (nkept == 0) {\n        for",
                                     "        double z = load_elem(x, c, dtype);\n        if (z > mu) mu = z;\n        ++nkept;\n    }\n    if (nkept == 0) {\n        for"),
    "variant_backward_sign": ("(load_elem(g, c, dtype) - dot)", "(load_elem(g, c, dtype) + dot)"),
    # attention
    "attention_diagonal_dropped": ("for (int64_t c = 0; c <= r; ++c) {\n        double dot = 0.0;",
                                   "for (int64_t c = 0; c < r; ++c) {\n        double dot = 0.0;"),
    "attention_scale_dropped": ("z[c] = scale * dot;", "z[c] = dot;"),
    "attention_key_transposed": ("load_elem(k, c * D + d, dtype);",
                                 "load_elem(k, d * (r + 1) + c, dtype);"),
    "attention_padded_rows_kept": ("    if (r >= L) return;\n    /* scores", "    if (r >= L + 1) return;\n    /* scores"),
    "attention_value_row_of_query": ("o[d] += p * load_elem(v, c * D + d, dtype);",
                                     "o[d] += p * load_elem(v, r * D + d, dtype);"),
    "variant_backward_dot_unmasked": ("if (keep[c]) dot += load_elem(g, c, dtype) * load_elem(y, c, dtype);",
                                      "dot += load_elem(g, c, dtype) * load_elem(y, c, dtype);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    lib = oracle.build(str(path), str(tmp_path / f"libmut_{name}.so"))
    orc = oracle.Oracle(lib)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception:  # any failure of a pin counts as caught
            failures.append(pin.__name__)
    assert failures, f"no pin catches mutation {name}"
