"""The oracle's pins catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a transposed
operand, a dropped term, a wrong index or sign, a wrong adapter), compiles
the copy with gcc into a temporary directory and runs every pin on it.  At
least one pin must fail for every planted mistake; the real oracle is never
modified.
"""
import os

import pytest

import oracle
import oracle_pins

# (name, text in the source, replacement, which occurrence (0-based) or None for all)
MUTANTS = [
    ("A_transposed", "A[h * r + k]", "A[k * H1 + h]", None),
    ("B_transposed", "B[k * H2 + j]", "B[j * r + k]", None),
    ("scale_dropped", "y[i * H2 + j] + scale * acc", "y[i * H2 + j] + acc", None),
    ("sign_flipped", "y[i * H2 + j] + scale * acc", "y[i * H2 + j] - scale * acc", None),
    ("y0_ignored", "y[i * H2 + j] = y[i * H2 + j] + scale * acc", "y[i * H2 + j] = scale * acc", None),
    ("shrink_uses_segment_not_adapter", "const int64_t a = adapter_ids[s];", "const int64_t a = s;", 0),
    ("expand_uses_segment_not_adapter", "const int64_t a = adapter_ids[s];", "const int64_t a = s;", 1),
    ("last_h_dropped", "h < H1; ++h", "h < H1 - 1; ++h", None),
    ("last_k_dropped", "k < r; ++k)\n                    acc", "k < r - 1; ++k)\n                    acc", None),
    ("segment_local_x_row", "x[i * H1 + h]", "x[(i - seg_indptr[s]) * H1 + h]", None),
    ("segment_end_off_by_one", "i < seg_indptr[s + 1]; ++i", "i < seg_indptr[s + 1] - 1; ++i", None),
    ("first_segment_skipped", "for (int32_t s = 0; s < num_segments; ++s) {\n        const", "for (int32_t s = 1; s < num_segments; ++s) {\n        const", None),
    ("v_k_reversed", "v[i * r + k] * (double)B", "v[i * r + (r - 1 - k)] * (double)B", None),
    ("adapter_stride_wrong", "a * (int64_t)H1 * r", "a * (int64_t)H1", None),
    ("y_not_initialised", "y[e] = (double)y0[e];", "y[e] = 0.0;", None),
    ("v_row_stride_wrong", "v[i * r + k] = acc;", "v[i + k] = acc;", None),
    ("W_transposed", "(double)wr[h]", "(double)W[h * H2 + j]", None),
    ("W_row_of_input", "W + j * (int64_t)H1", "W + i * (int64_t)H1", None),
    ("linear_bias_dropped", "acc + (double)bias[j]", "acc", None),
    ("linear_bias_wrong_index", "(double)bias[j]", "(double)bias[0]", None),
    ("linear_x_row_zero", "x + i * (int64_t)H1", "x", None),
    ("linear_addon_skipped", "if (!rc)\n        rc = sgmv_oracle_expand", "if (0)\n        rc = sgmv_oracle_expand", None),
    ("linear_base_sign_flipped", "y[i * H2 + j] = bias ? acc", "y[i * H2 + j] = bias ? -acc", None),
]


def _plant(src, old, new, which):
    assert old in src, f"mutation anchor not found: {old!r}"
    if which is None:
        return src.replace(old, new)
    parts = src.split(old)
    assert len(parts) > which + 1
    return old.join(parts[:which + 1]) + new + old.join(parts[which + 1:])


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, which):
    with open(oracle.SOURCE) as f:
        src = f.read()
    mutated = _plant(src, old, new, which)
    assert mutated != src
    c_path = os.path.join(tmp_path, f"{name}.c")
    with open(c_path, "w") as f:
        f.write(mutated)
    so = oracle.build(c_path, os.path.join(tmp_path, f"lib{name}.so"))
    mutant = oracle.Oracle(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
