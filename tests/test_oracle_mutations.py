"""The oracle's pins are sensitive: plant plausible mistakes in a copy of the
oracle source (on the CPU) and check that at least one pin fails for each.

Each mutant is a textual edit of ``oracle/oracle.c`` compiled into a
temporary library; the pins run against it in place of the real oracle.
"""
import ctypes
import os

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, mutated text, pins expected to catch it)
MUTANTS = [
    ("dq_missing_scale", "dqi[cc] += scale * ds[j] * k[j * d + cc]",
     "dqi[cc] += ds[j] * k[j * d + cc]",
     [lambda: pins.test_matches_torch_cpu_fp64_sdpa_and_autograd(17, 8, False)]),
    ("ds_wrong_sign", "ds[j] = prob[j] * (dp - Di);", "ds[j] = prob[j] * (dp + Di);",
     [lambda: pins.test_gradient_sum_identities(False, 0.0)]),
    ("dk_transposed_operand", "dkj[cc] += scale * dsij * q[i * d + cc];",
     "dkj[cc] += scale * dsij * q[j * d + cc];",
     [lambda: pins.test_gradients_match_finite_differences(3, 4, False, 0.0)]),
    ("causal_off_by_one", "if (causal && j > i) { s[j] = -INFINITY; continue; }",
     "if (causal && j >= i && i > 0) { s[j] = -INFINITY; continue; }",
     [lambda: pins.test_zero_query_gives_mean_of_values(True)]),
    ("bwd_dropout_scale_dropped", "double dp = dpd * keep * c;", "double dp = dpd * keep;",
     [lambda: pins.test_gradients_match_finite_differences(5, 2, True, 0.5)]),
    ("fwd_dropout_not_rescaled", "pd[j] = keep_bit(seed, b, h, i, j, T) ? pij * c : 0.0;",
     "pd[j] = keep_bit(seed, b, h, i, j, T) ? pij : 0.0;",
     [pins.test_dropout_is_unbiased]),
    ("lse_without_log", "return m + log(l);", "return m + l;",
     [lambda: pins.test_zero_query_gives_mean_of_values(False)]),
    ("scale_dropped_in_scores", "s[j] = scale * acc;", "s[j] = acc;",
     [lambda: pins.test_key_shift_invariance(False)]),
    ("keep_threshold_inverted", "return v16 >= T;", "return v16 < T;",
     [pins.test_dropout_kept_fraction_within_five_sigma]),
    ("value_row_index_swapped", "for (int64_t c = 0; c < d; ++c) oi[c] += pd[j] * vj[c];",
     "for (int64_t c = 0; c < d; ++c) oi[c] += pd[j] * v[i * d + c];",
     [lambda: pins.test_one_hot_values_select_probabilities(False, 0.0)]),
    ("cross_causal_offset_sign", "const int64_t last = causal ? i + (Nk - Nq) : Nk - 1;",
     "const int64_t last = causal ? i - (Nk - Nq) : Nk - 1;",
     [lambda: pins.test_cross_causal_is_the_tail_of_the_square_problem(1, 40)]),
    ("cross_last_key_dropped", "const int64_t last = causal ? i + (Nk - Nq) : Nk - 1;",
     "const int64_t last = causal ? i + (Nk - Nq) : Nk - 2;",
     [lambda: pins.test_cross_matches_torch_cpu_fp64_sdpa(5, 23, False)]),
    ("cross_dropout_row_shifted", "prob_row(Nk, s, lse, p, seed, b, h, i, prob, pd);",
     "prob_row(Nk, s, lse, p, seed, b, h, i + (Nk - Nq), prob, pd);",
     [pins.test_cross_dropout_uses_the_square_counters]),
    ("cross_bwd_dropout_scale_dropped", "ds[j] = prob[j] * (dpd * keep * c - Di);",
     "ds[j] = prob[j] * (dpd * keep - Di);",
     [lambda: pins.test_cross_gradients_match_finite_differences(3, 6, 2, True, 0.5)]),
    ("cross_bwd_dk_row_index", "dkj[cc] += dsij * scale * q[i * d + cc];",
     "dkj[cc] += dsij * scale * q[(Nq - 1 - i) * d + cc];",
     [lambda: pins.test_cross_gradients_match_torch_fp64_autograd(5, 23, False)]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, checks, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found once: %r" % old
    mutant_c = tmp_path / ("%s.c" % name)
    mutant_c.write_text(src.replace(old, new))
    so = oracle.compile_source(str(mutant_c), str(tmp_path / ("lib%s.so" % name)))
    lib = oracle._bind(ctypes.CDLL(so))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught == len(checks), "mutant %s survived its pins" % name
