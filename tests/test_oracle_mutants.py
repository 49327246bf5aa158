"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of ``oracle/ets_oracle.c`` with one plausible mistake
planted (on the CPU only), compiled to its own library; the pin tests of this
suite are then run against it and at least one of them has to fail.
"""
import contextlib
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_bruteforce as tb
from tests import test_oracle_closed_forms as tc

SRC = os.path.join(os.path.dirname(oracle.__file__), "ets_oracle.c")

MUTANTS = {
    "tie_break_reversed": ("if (x->pos != y->pos) return (x->pos < y->pos) ? -1 : 1;",
                           "if (x->pos != y->pos) return (x->pos > y->pos) ? -1 : 1;"),
    "ascending_keys": ("if (x->key != y->key) return (x->key > y->key) ? -1 : 1;",
                       "if (x->key != y->key) return (x->key < y->key) ? -1 : 1;"),
    "negatives_not_inverted": ("if (bits & 0x80000000u) return ~bits;",
                               "if (bits & 0x80000000u) return bits & 0x7FFFFFFFu;"),
    "sign_bit_not_set": ("return bits | 0x80000000u;", "return bits;"),
    "page_and_slot_swapped": ("const int32_t page = i / job->page_size;",
                              "const int32_t page = i % job->page_size;"),
    "padding_not_written": ("for (int32_t j = m; j < job->k; ++j) out_row[j] = -1;",
                            "for (int32_t j = m; j < job->k; ++j) out_row[j] = 0;"),
    "one_short": ("const int32_t m = n < job->k ? n : job->k;",
                  "const int32_t m = n < job->k ? n : job->k - 1;"),
    "no_upper_clamp": ("if (n > job->L) n = job->L;", ""),
    "ragged_offset_dropped": ("v = job->row_starts[b] + i;", "v = i;"),
}


@contextlib.contextmanager
def _swapped(lib):
    saved = oracle._lib
    oracle._lib = lib
    try:
        yield
    finally:
        oracle._lib = saved


def _run_pins():
    """Run the pin tests against whatever library ``oracle`` currently uses."""
    with open(tc.GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        tc.test_golden_hand_rows(oracle, case)
    for n in range(0, 5):
        tb.test_all_rows_over_alphabet(oracle, n)
    tc.test_all_equal_takes_lowest_positions(oracle, 100, 7)
    tc.test_monotone_rows(oracle, 10, 3)
    tc.test_planted_maxima(oracle)
    tc.test_lengths_clamp_and_poisoned_tail(oracle)
    tc.test_paged_identity_equals_raw(oracle)
    tc.test_paged_permuted_table_closed_form(oracle, 64)
    tc.test_ragged_matches_rows(oracle)


def test_pins_pass_on_real_oracle(oracle_mod):
    _run_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: %s" % name
    mpath = tmp_path / ("mutant_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    so = str(tmp_path / ("libmutant_%s.so" % name))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(mpath),
                    "-o", so], check=True)
    lib = oracle._bind(so)
    with _swapped(lib):
        with pytest.raises((AssertionError, RuntimeError)):
            _run_pins()
    assert np.all(oracle.topk_raw(np.arange(4, dtype=np.float32)[None], 2) == [[3, 2]])
