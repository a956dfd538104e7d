"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a text substitution in a temporary copy of qmm_oracle.c,
compiled with gcc and loaded in place of the real oracle for the duration of
the test.  The real oracle's source is never modified.
"""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "qmm_oracle.c")

# (name, original text, replacement, how many occurrences to replace (0 = all))
MUTANTS = [
    ("drop_min", "double wv = s * (double)row_code(row, c, bits) + m;",
     "double wv = s * (double)row_code(row, c, bits);", 1),
    ("min_sign", "double wv = s * (double)row_code(row, c, bits) + m;",
     "double wv = s * (double)row_code(row, c, bits) - m;", 1),
    ("group_index_mod", "scales[r * gpr + c / group]", "scales[r * gpr + c % group]", 0),
    ("scale_min_swapped", "double s = qmo_fp16_to_double(scales[r * gpr + c / group]);\n"
     "                double m = qmo_fp16_to_double(mins[r * gpr + c / group]);\n"
     "                double wv",
     "double s = qmo_fp16_to_double(mins[r * gpr + c / group]);\n"
     "                double m = qmo_fp16_to_double(scales[r * gpr + c / group]);\n"
     "                double wv", 1),
    ("msb_first_codes", "q |= row_bit(row, k * bits + j) << j;",
     "q |= row_bit(row, k * bits + j) << (bits - 1 - j);", 1),
    ("word_bit_reversed", "return (row[i / 32] >> (i % 32)) & 1u;",
     "return (row[i / 32] >> (31 - i % 32)) & 1u;", 1),
    ("pack_bit_reversed", "row[i / 32] |= (uint32_t)((q >> j) & 1u) << (i % 32);",
     "row[i / 32] |= (uint32_t)((q >> j) & 1u) << (31 - i % 32);", 1),
    ("x_off_by_one", "double p = wv * qmo_fp16_to_double(xr[c]);",
     "double p = wv * qmo_fp16_to_double(xr[(c + 1) % k]);", 1),
    ("x_row_ignored", "const uint16_t *xr = x + (x_rows ? (int64_t)x_rows[i] : i) * k;",
     "const uint16_t *xr = x;", 1),
    ("fp16_bias", "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);", 1),
    ("fp16_subnormal", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);", 1),
    ("fp16_no_sign", "return s ? -v : v;", "return v;", 1),
    ("abs_sum_signed", "acc_abs += fabs(p);", "acc_abs += p;", 0),
    ("moe_expert_stride", "int64_t w_expert = n * words_per_row(k, bits);",
     "int64_t w_expert = (n - 1) * words_per_row(k, bits);", 1),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(mutant, tmp_path):
    name, old, new, count = mutant
    text = open(SRC).read()
    assert old in text, "mutation anchor not found: %s" % name
    text = text.replace(old, new) if count == 0 else text.replace(old, new, count)
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(text)
    lib = str(tmp_path / ("libmutant_%s.so" % name))
    oracle.compile_source(str(src), lib)
    failed = []
    oracle.use_library(lib)
    try:
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except AssertionError:
                failed.append(check.__name__)
    finally:
        oracle.use_library(None)
    assert failed, "planted mistake %r passed every pin" % name


# Planted mistakes in the fp16-weight path (Python): each replaces one oracle
# function for the duration of the test and must fail at least one pin.
def _f16_halves_swapped(w_words, n, k):
    import numpy as np
    w = oracle._c(w_words, np.uint32).reshape(n, k // 2)
    h = np.empty((n, k), dtype=np.uint16)
    h[:, 0::2] = (w >> 16).astype(np.uint16)
    h[:, 1::2] = (w & 0xFFFF).astype(np.uint16)
    return oracle.fp16_to_double(h)


def _f16_as_integers(w_words, n, k):
    # Reads the 16-bit patterns as integers instead of decoding them.
    import numpy as np
    w = oracle._c(w_words, np.uint32).reshape(n, k // 2)
    h = np.empty((n, k), dtype=np.float64)
    h[:, 0::2] = w & 0xFFFF
    h[:, 1::2] = w >> 16
    return h


_real_qmm_f16 = oracle._qmm_f16


def _qmm_f16_abs_signed(w_words, x2, n, k):
    y, _ = _real_qmm_f16(w_words, x2, n, k)
    return y, y


def _qmm_f16_x_shifted(w_words, x2, n, k):
    import numpy as np
    return _real_qmm_f16(w_words, np.roll(x2, 1, axis=1), n, k)


_real_moe_combine = oracle.moe_combine


def _combine_by_pair_index(y_pair, a_pair, pair_token, pair_weight, n_tokens, y0=None):
    # Sends pair p to row p % n_tokens instead of its token's row.
    import numpy as np
    tok = np.arange(len(pair_token), dtype=np.int32) % n_tokens
    return _real_moe_combine(y_pair, a_pair, tok, pair_weight, n_tokens, y0)


def _combine_unweighted(y_pair, a_pair, pair_token, pair_weight, n_tokens, y0=None):
    import numpy as np
    return _real_moe_combine(y_pair, a_pair, pair_token, np.ones(len(pair_token)), n_tokens, y0)


def _combine_drops_y0(y_pair, a_pair, pair_token, pair_weight, n_tokens, y0=None):
    return _real_moe_combine(y_pair, a_pair, pair_token, pair_weight, n_tokens, None)


def _combine_weight_order_reversed(y_pair, a_pair, pair_token, pair_weight, n_tokens, y0=None):
    return _real_moe_combine(y_pair, a_pair, pair_token, pair_weight[::-1], n_tokens, y0)


PY_MUTANTS = [
    ("combine_by_pair_index", "moe_combine", _combine_by_pair_index),
    ("combine_unweighted", "moe_combine", _combine_unweighted),
    ("combine_drops_y0", "moe_combine", _combine_drops_y0),
    ("combine_weights_reversed", "moe_combine", _combine_weight_order_reversed),
    ("f16_halves_swapped", "f16_weights", _f16_halves_swapped),
    ("f16_not_decoded", "f16_weights", _f16_as_integers),
    ("f16_abs_sum_signed", "_qmm_f16", _qmm_f16_abs_signed),
    ("f16_x_off_by_one", "_qmm_f16", _qmm_f16_x_shifted),
]


@pytest.mark.parametrize("mutant", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_python_mistake_is_caught(mutant, monkeypatch):
    name, attr, fn = mutant
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "planted mistake %r passed every pin" % name
