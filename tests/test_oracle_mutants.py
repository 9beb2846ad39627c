"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch each one: a dropped term, a wrong sign, a wrong index or
layout, a transposed operand, a swapped order of update and readout.

Each mutant is compiled from the oracle's source text with one replacement,
bound through the same wrapper, and run against a fixed subset of the pins;
at least one pin must fail.  The real oracle is never modified.
"""
import pytest

import oracle
import test_oracle_golden as G
import test_oracle_pins as P

MUTANTS = [
    ("A_sign", "A[n] = -exp(A_log[d * dstate + n]);", "A[n] = exp(A_log[d * dstate + n]);"),
    ("A_ignored_in_decay", "double Abar = exp(dA);", "double Abar = exp(-Delta);"),
    ("u_dropped", "h[n] = Abar * h[n] + Bbar * u;", "h[n] = Abar * h[n] + Bbar;"),
    ("readout_before_update",
     "h[n] = Abar * h[n] + Bbar * u;\n    acc += Ct[n * c_stride] * h[n];",
     "acc += Ct[n * c_stride] * h[n];\n    h[n] = Abar * h[n] + Bbar * u;"),
    ("D_dropped", "double y = acc + Dd * u;", "double y = acc;"),
    ("gate_before_D",
     "double y = acc + Dd * u;\n  if (zt) y = y * oracle_silu(*zt);",
     "double y = acc;\n  if (zt) y = y * oracle_silu(*zt);\n  y += Dd * u;"),
    ("bias_dropped", "double x = dlt + bias;", "double x = dlt;"),
    ("euler_bbar", "expm1(dA) / A[n] * Bn", "Delta * Bn"),
    ("A_log_transposed", "A_log[d * dstate + n]", "A_log[n * dim + d]"),
    ("B_layout_time_major", "B + bcrow + t, seqlen", "B + bcrow + t * dstate, 1"),
    ("C_reads_B", "C + bcrow + t, seqlen, Dd", "B + bcrow + t, seqlen, Dd"),
    ("B_batch_ignored", "const int64_t bcrow = b * dstate * seqlen;", "const int64_t bcrow = 0;"),
    ("initial_state_ignored", "h[n] = initial_state ? initial_state[bd * dstate + n] : 0.0;", "h[n] = 0.0;"),
    ("softplus_missing_linear_part", "return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));",
     "return log1p(exp(-fabs(x)));"),
    ("silu_is_sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("step_dt_bias_dropped", "dt_bias ? dt_bias[d] : 0.0", "0.0"),
    ("step_B_batch_ignored", "B + b * dstate, 1, C + b * dstate, 1", "B, 1, C + b * dstate, 1"),
]

PINS = [
    G.test_theorem1_gated_rnn,
    G.test_lti_one_state,
    G.test_lti_two_states,
    G.test_delta_zero_persist,
    G.test_delta_large_reset,
    G.test_step_one_token,
    lambda o: P.test_products_vanloan(o, (2, 3, 4, 8), True, True, True),
    lambda o: P.test_products_vanloan(o, (2, 3, 4, 8), False, False, False),
    lambda o: P.test_theorem1_vs_expit(o, 1),
    P.test_d_skip_alone,
    P.test_gate_matches_torch_silu,
    lambda o: P.test_split_resume_every_k(o, True),
    lambda o: P.test_chained_steps_equal_scan(o, True, True),
    lambda o: P.test_chained_steps_equal_scan(o, False, False),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert old in src, f"mutation site for {name} not found"
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path), "mut_" + name)
    caught = []
    for pin in PINS:
        try:
            pin(variant)
        except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path):
    variant = oracle.build_variant(oracle.source_text(), str(tmp_path), "copy")
    for pin in PINS:
        pin(variant)
