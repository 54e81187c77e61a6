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
    "backward_scale_dropped": ("dx[off + c] = (double)scale * load_elem(y, off + c, dtype) *",
                               "dx[off + c] = load_elem(y, off + c, dtype) *"),
    "row_column_swapped": ("if (kept(r, c, L))\n            y[c]",
                           "if (kept(c, r, L))\n            y[c]"),
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
