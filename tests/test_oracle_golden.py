"""Oracle vs. hand-derived worked examples (tests/golden/*.json).

The pages print no numeric worked example, so each fixture is a small case
whose answer follows by hand from a formula the pages state (ZOH, the
convolution dual, Theorem 1, the Delta limits); the fixture carries the
citation and the derivation.  Not from the oracle.
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name + ".json")) as f:
        return json.load(f)


def _close(got, exp, tol):
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    assert got.shape == exp.shape
    if tol == 0.0:
        assert np.array_equal(got, exp), (got, exp)
    else:
        assert np.max(np.abs(got - exp) / np.maximum(np.abs(exp), 1.0)) <= tol, (got, exp)


def test_theorem1_gated_rnn(oracle_mod):
    fx = _load("theorem1_gated_rnn")
    for case in fx["cases"]:
        L = len(case["u"])
        u = np.array(case["u"]).reshape(1, 1, L)
        dl = np.array(case["delta"]).reshape(1, 1, L)
        y, fs = oracle_mod.scan_fwd(u, dl, np.zeros((1, 1)), np.ones((1, 1, L)), np.ones((1, 1, L)),
                                    delta_bias=np.array([case["bias"]]), delta_softplus=True)
        _close(y.ravel(), case["expected_y"], fx["tol"])
        _close(fs.ravel(), [case["expected_final"]], fx["tol"])


def test_lti_one_state(oracle_mod):
    fx = _load("lti_one_state")
    L = len(fx["u"])
    u = np.array(fx["u"]).reshape(1, 1, L)
    dl = np.array(fx["delta"]).reshape(1, 1, L)
    args = dict(u=u, delta=dl, A_log=np.zeros((1, 1)), B=np.full((1, 1, L), fx["B"]),
                C=np.full((1, 1, L), fx["C"]), D=np.array([fx["D"]]), delta_softplus=False)
    y, fs = oracle_mod.scan_fwd(**args)
    _close(y.ravel(), fx["expected_y"], fx["tol"])
    _close(fs.ravel(), [fx["expected_final"]], fx["tol"])
    yg, _ = oracle_mod.scan_fwd(z=np.full((1, 1, L), fx["z_const"]), **args)
    _close(yg.ravel(), np.array(fx["expected_y"]) * fx["silu_z"], fx["tol"])


def test_lti_two_states(oracle_mod):
    fx = _load("lti_two_states")
    L = len(fx["u"])
    B = np.array(fx["B"]).reshape(1, 2, 1).repeat(L, axis=2)
    C = np.array(fx["C"]).reshape(1, 2, 1).repeat(L, axis=2)
    y, fs = oracle_mod.scan_fwd(np.array(fx["u"]).reshape(1, 1, L), np.array(fx["delta"]).reshape(1, 1, L),
                                np.array(fx["A_log"]).reshape(1, 2), B, C, delta_softplus=False)
    _close(y.ravel(), fx["expected_y"], fx["tol"])
    _close(fs.ravel(), fx["expected_final"], fx["tol"])


def test_delta_zero_persist(oracle_mod):
    fx = _load("delta_zero_persist")
    L = len(fx["u"])
    y, fs = oracle_mod.scan_fwd(np.array(fx["u"]).reshape(1, 1, L), np.zeros((1, 1, L)),
                                np.array(fx["A_log"]).reshape(1, 2), np.array(fx["B"]).reshape(1, 2, L),
                                np.array(fx["C"]).reshape(1, 2, L), D=np.array([fx["D"]]),
                                initial_state=np.array(fx["h0"]).reshape(1, 1, 2), delta_softplus=False)
    _close(y.ravel(), fx["expected_y"], fx["tol"])
    _close(fs.ravel(), fx["expected_final"], fx["tol"])


def test_delta_large_reset(oracle_mod):
    fx = _load("delta_large_reset")
    L = len(fx["u"])
    y, fs = oracle_mod.scan_fwd(np.array(fx["u"]).reshape(1, 1, L), np.full((1, 1, L), fx["delta"]),
                                np.array(fx["A_log"]).reshape(1, 2), np.ones((1, 2, L)), np.ones((1, 2, L)),
                                delta_softplus=False)
    _close(y.ravel(), fx["expected_y"], fx["tol"])
    _close(fs.ravel(), fx["expected_final"], fx["tol"])


def test_step_one_token(oracle_mod):
    fx = _load("step_one_token")
    args = dict(state=np.array(fx["state"]).reshape(1, 1, 2), x=np.array([[fx["x"]]]), dt=np.array([[fx["dt"]]]),
                A_log=np.array(fx["A_log"]).reshape(1, 2), B=np.array(fx["B"]).reshape(1, 2),
                C=np.array(fx["C"]).reshape(1, 2), D=np.array([fx["D"]]), dt_softplus=False)
    y, st = oracle_mod.scan_step(**args)
    _close(y.ravel(), [fx["expected_y"]], fx["tol"])
    _close(st.ravel(), fx["expected_state"], fx["tol"])
    yg, _ = oracle_mod.scan_step(z=np.array([[fx["z"]]]), **args)
    _close(yg.ravel(), [fx["expected_y_gated"]], fx["tol"])
