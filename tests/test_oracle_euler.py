"""Pins of the oracle's Euler variant (Bbar = Delta B; Mamba notes, 设计 1
pseudo-code, the input term written as Delta B x), each derived by a route
that shares nothing with the oracle's loop:

* a closed form: one state with constant inputs is a geometric series;
* the Euler and zero-order-hold input terms differ at second order in Delta,
  by A Delta^2 / 2 times B u (Taylor expansion of expm1);
* the products form h_t = sum_j (prod_{s=j+1..t} Abar_s) Delta_j B_j u_j with
  Abar = exp(Delta A), written out in numpy, at random multi-state inputs with
  gate, D skip, bias and initial state;
* chained Euler steps equal the Euler scan bit for bit;
* planted mistakes in copies of the oracle are caught.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)


def _case(b, d, n, L, rng, gated=True):
    return dict(u=rng.standard_normal((b, d, L)), delta=rng.standard_normal((b, d, L)) * 0.7 - 0.5,
                A_log=rng.uniform(-1.0, 1.5, size=(d, n)), B=rng.standard_normal((b, n, L)),
                C=rng.standard_normal((b, n, L)), D=rng.standard_normal(d),
                z=rng.standard_normal((b, d, L)) if gated else None, delta_bias=rng.uniform(-1.0, 0.5, size=d),
                initial_state=rng.standard_normal((b, d, n)) * 0.3)


def test_euler_geometric_closed_form(o=oracle):
    """N = 1, constant Delta, A, B, u and C = 1, no D, no gate: h_t = a h_{t-1} + Delta B u with
    a = exp(Delta A), so h_t = Delta B u (1 - a^(t+1)) / (1 - a) from h_{-1} = 0."""
    L, Delta, A, Bv, uv = 12, 0.3, -0.8, 1.7, -0.6
    a = np.exp(Delta * A)
    u = np.full((1, 1, L), uv)
    delta = np.full((1, 1, L), Delta)
    A_log = np.array([[np.log(-A)]])
    B = np.full((1, 1, L), Bv)
    C = np.ones((1, 1, L))
    y, fs = o.scan_fwd(u, delta, A_log, B, C, delta_softplus=False, discretization="euler")
    t = np.arange(L)
    want = Delta * Bv * uv * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(y[0, 0], want, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fs[0, 0, 0], want[-1], rtol=1e-13)


@pytest.mark.parametrize("Delta", [1e-2, 1e-3])
def test_euler_vs_zoh_second_order(Delta, o=oracle):
    """One token from a zero state, no D, no gate: y = C Bbar u.  ZOH has Bbar = expm1(Delta A)/A B,
    Euler Delta B, so (y_zoh - y_euler) / Delta^2 -> A C B u / 2 with a relative error O(Delta)."""
    n = 3
    A = -np.array([0.5, 1.0, 2.5])
    Bv = np.array([0.7, -1.2, 0.4])
    Cv = np.array([1.1, 0.3, -0.9])
    uv = 0.8
    args = dict(u=np.full((1, 1, 1), uv), delta=np.full((1, 1, 1), Delta), A_log=np.log(-A)[None, :],
                B=Bv.reshape(1, n, 1), C=Cv.reshape(1, n, 1), delta_softplus=False)
    yz, _ = o.scan_fwd(**args, discretization="zoh")
    ye, _ = o.scan_fwd(**args, discretization="euler")
    np.testing.assert_allclose(ye[0, 0, 0], Delta * uv * np.dot(Cv, Bv), rtol=1e-14)
    lead = uv * np.dot(Cv * A, Bv) / 2
    got = (yz[0, 0, 0] - ye[0, 0, 0]) / Delta ** 2
    assert abs(got - lead) <= 2 * Delta * abs(uv) * np.dot(np.abs(Cv * A * A), np.abs(Bv)) / 6 + 1e-9


def _products_euler(c):
    u, C = c["u"], c["C"]
    b_, d_, L = u.shape
    n_ = c["A_log"].shape[1]
    Delta = np.logaddexp(0.0, c["delta"] + c["delta_bias"][None, :, None])
    A = -np.exp(c["A_log"])
    y = np.zeros((b_, d_, L))
    hL = np.zeros((b_, d_, n_))
    for b in range(b_):
        for d in range(d_):
            logA = Delta[b, d][:, None] * A[d][None, :]                      # (L, n): log Abar_t
            cum = np.concatenate([np.zeros((1, n_)), np.cumsum(logA, axis=0)])  # cum[t+1] = sum_{s<=t}
            for t in range(L):
                h = np.exp(cum[t + 1]) * c["initial_state"][b, d]
                for j in range(t + 1):
                    h = h + np.exp(cum[t + 1] - cum[j + 1]) * Delta[b, d, j] * c["B"][b, :, j] * u[b, d, j]
                yt = np.dot(C[b, :, t], h) + c["D"][d] * u[b, d, t]
                if c["z"] is not None:
                    zt = c["z"][b, d, t]
                    yt *= zt / (1 + np.exp(-zt))
                y[b, d, t] = yt
                if t == L - 1:
                    hL[b, d] = h
    return y, hL


@pytest.mark.parametrize("shape", [(1, 1, 1, 5), (2, 3, 4, 9)])
def test_euler_products_form(shape, o=oracle):
    c = _case(*shape, np.random.default_rng(sum(shape)))
    y, fs = o.scan_fwd(**c, discretization="euler")
    yr, hr = _products_euler(c)
    np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fs, hr, rtol=1e-10, atol=1e-12)


def test_euler_chained_steps_equal_scan(o=oracle):
    c = _case(2, 3, 4, 7, np.random.default_rng(5))
    y, fs = o.scan_fwd(**c, discretization="euler")
    st = c["initial_state"].copy()
    for t in range(7):
        yt, st = o.scan_step(st, c["u"][..., t], c["delta"][..., t], c["A_log"], c["B"][..., t], c["C"][..., t],
                             D=c["D"], z=c["z"][..., t], dt_bias=c["delta_bias"], discretization="euler")
        assert np.array_equal(yt, y[..., t])
    assert np.array_equal(st, fs)


def test_euler_and_zoh_differ(o=oracle):
    c = _case(1, 2, 3, 6, np.random.default_rng(8))
    yz, _ = o.scan_fwd(**c)
    ye, _ = o.scan_fwd(**c, discretization="euler")
    assert np.max(np.abs(yz - ye)) > 1e-3


def test_bad_discretization_rejected():
    c = _case(1, 1, 1, 2, np.random.default_rng(1))
    with pytest.raises(ValueError):
        oracle.scan_fwd(**c, discretization="bilinear")


EULER_MUTANTS = [
    ("euler_uses_zoh", "Bbar = Delta * Bn;                                            /* Euler input term */",
     "Bbar = expm1(dA) / A[n] * Bn;"),
    ("euler_drops_delta", "Bbar = Delta * Bn;                                            /* Euler input term */",
     "Bbar = Bn;"),
    ("euler_flag_ignored_in_step", "dt_softplus, euler, B + b * dstate, 1,", "dt_softplus, 0, B + b * dstate, 1,"),
]

EULER_PINS = [
    test_euler_geometric_closed_form,
    lambda o: test_euler_vs_zoh_second_order(1e-2, o),
    lambda o: test_euler_products_form((2, 3, 4, 9), o),
    test_euler_chained_steps_equal_scan,
]


@pytest.mark.parametrize("name,old,new", EULER_MUTANTS, ids=[m[0] for m in EULER_MUTANTS])
def test_euler_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert old in src, f"mutation site for {name} not found"
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path), "mut_" + name)
    caught = 0
    for pin in EULER_PINS:
        try:
            pin(variant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught, f"no pin caught the planted mistake {name}"
