"""Mutation check of the oracle's pins, on the CPU.

Each case plants one plausible mistake in a private copy of the oracle's C
source (a dropped term, a wrong sign, a transposed operand, a lost stride,
alpha in the wrong place, single-precision accumulation, ...), builds it, and
requires that at least one pin rejects it.  The unmodified source must pass
every pin.  Nothing here touches the product library.
"""
import functools
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ref_sgemm.c")

MUTANTS = {
    "drop_last_term": [("for (int64_t p = 0; p < k; ++p)", "for (int64_t p = 0; p < k - 1; ++p)")],
    "drop_first_term": [("for (int64_t p = 0; p < k; ++p)", "for (int64_t p = 1; p < k; ++p)")],
    "wrong_sign": [("sum += a * bv;", "sum -= a * bv;")],
    "transposed_A": [("elem_offset(b, i, p, sA_batch, sA_row, sA_col)",
                      "elem_offset(b, p, i, sA_batch, sA_row, sA_col)")],
    "transposed_B": [("elem_offset(b, p, j, sB_batch, sB_row, sB_col)",
                      "elem_offset(b, j, p, sB_batch, sB_row, sB_col)")],
    "strides_exchanged": [("return b * s_batch + r * s_row + c * s_col;",
                           "return b * s_batch + r * s_col + c * s_row;")],
    "alpha_dropped": [("double out = (double)alpha * total;", "double out = total;")],
    "alpha_on_c_old": [("out += (double)beta * (double)*c_old;", "out += (double)alpha * (double)*c_old;")],
    "accumulate_inverted": [("return accumulate ? 1.0f : 0.0f;", "return accumulate ? 0.0f : 1.0f;")],
    "always_accumulate": [("return accumulate ? 1.0f : 0.0f;", "return 1.0f;")],
    "fp32_accumulation": [("double sum = 0.0;", "float sum = 0.0f;")],
    "batch_row_swapped": [("int64_t b = row / m, i = row % m;", "int64_t b = row % m, i = row / m;")],
    "B_batch_ignored": [("elem_offset(b, p, j, sB_batch", "elem_offset(0, p, j, sB_batch")],
    "last_column_skipped": [("for (int64_t jj = 0; jj < n; ++jj)", "for (int64_t jj = 0; jj < n - 1; ++jj)")],
    "alpha_rounded_to_int": [("double out = (double)alpha * total;", "double out = (double)(int)alpha * total;")],
    "beta_ignored": [("out += (double)beta * (double)*c_old;", "out += (double)*c_old;")],
    "c_old_read_at_beta_zero": [("if (beta != 0.0f)", "if (1)")],
    "row_term_dropped": [("out += (double)row_add[b * sR_batch + i * sR_row];", "out += 0.0;")],
    "col_term_dropped": [("out += (double)col_add[b * sL_batch + j * sL_col];", "out += 0.0;")],
    "row_term_by_column": [("row_add[b * sR_batch + i * sR_row]", "row_add[b * sR_batch + j * sR_row]")],
    "vector_batch_ignored": [("col_add[b * sL_batch + j * sL_col]", "col_add[j * sL_col]")],
    "norm_not_squared": [("sq += x * x;", "sq += x;")],
    "norm_last_element_skipped": [("for (int64_t e = 0; e < len; ++e)", "for (int64_t e = 0; e < len - 1; ++e)")],
    "distance_sum_not_difference": [("(double)X[bq * sX_batch + iq * sX_row + e * sX_col] -",
                                     "(double)X[bq * sX_batch + iq * sX_row + e * sX_col] +")],
    "distance_Y_transposed": [("(double)Y[bq * sY_batch + jq * sY_row + e * sY_col]",
                               "(double)Y[bq * sY_batch + e * sY_row + jq * sY_col]")],
    "distance_not_squared": [("d += diff * diff;", "d += diff < 0 ? -diff : diff;")],
    "kv_group_ignored": [("B + o * sB_outer + (i / gB) * sB_inner", "B + o * sB_outer + (i / 1) * sB_inner")],
    "group_of_the_wrong_operand": [("B + o * sB_outer + (i / gB) * sB_inner", "B + o * sB_outer + (i / gA) * sB_inner")],
    "batch_levels_swapped_in_C": [("C + o * sC_outer + i * sC_inner", "C + i * sC_outer + o * sC_inner")],
    "mask_off_by_one": [("causal ? q + (tk - tq) + 1 : tk", "causal ? (q + (tk - tq) + 2 < tk ? q + (tk - tq) + 2 : tk) : tk")],
    "mask_top_left": [("causal ? q + (tk - tq) + 1 : tk", "causal ? q + 1 : tk")],
    "no_max_subtraction": [("s[j] = exp(s[j] - mx);", "s[j] = exp(s[j]);")],
    "softmax_not_normalised": [("s[j] /= z;", "s[j] /= 1.0;")],
    "scores_without_alpha": [("s[j] = (double)alpha * dot;", "s[j] = dot;")],
    "softmax_max_of_first_key": [("if (s[j] > mx) mx = s[j];", "if (0) mx = s[j];")],
    "attention_V_transposed": [("Vb[j * sV_row + c * sV_col]", "Vb[c * sV_row + j * sV_col]")],
    "attention_K_at_query_row": [("Kb[j * sK_row + p * sK_col]", "Kb[q * sK_row + p * sK_col]")],
    "attention_kv_group_ignored_in_K": [("K + o * sK_outer + (i / g) * sK_inner", "K + o * sK_outer + (i % g) * sK_inner")],
    "attention_kv_group_ignored_in_V": [("V + o * sV_outer + (i / g) * sV_inner", "V + o * sV_outer + (i % g) * sV_inner")],
    "attention_last_dim_skipped": [("for (int64_t p = 0; p < d; ++p)", "for (int64_t p = 0; p < d - 1; ++p)")],
}

# The brute-force pin at full size is slow; mutants see a smaller sweep.
BATTERY = [p if p is not pins.pin_exact_bruteforce
           else functools.partial(pins.pin_exact_bruteforce, sizes=range(1, 5))
           for p in pins.PINS]


def _build(tmp_path, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    return oracle.build(str(path), str(tmp_path / "libmutant.so"))


def _first_failing_pin(lib):
    for pin in BATTERY:
        try:
            pin(lib)
        except AssertionError:
            return getattr(pin, "__name__", getattr(pin, "func", pin).__name__)
    return None


def _child(lib_path):
    """Runs in a fresh interpreter: the battery against one build."""
    return _first_failing_pin(oracle.load_library(lib_path))


def _outcome(tmp_path, edits):
    """Name of the first pin that rejects the build, "crash:<rc>" if the
    mutant brings its process down (an index mutation can read outside its
    buffer), or None if every pin passes."""
    lib_path = _build(tmp_path, edits)
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle_mutants as t; "
            "print('OUTCOME', t._child(%r))" % (here, root, lib_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return f"crash:{r.returncode}"
    line = [l for l in r.stdout.splitlines() if l.startswith("OUTCOME ")][-1]
    v = line.split(" ", 1)[1]
    return None if v == "None" else v


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    assert _outcome(tmp_path, MUTANTS[name]) is not None, f"no pin rejects mutant {name}"


def test_pristine_copy_passes(tmp_path):
    assert _outcome(tmp_path, []) is None
