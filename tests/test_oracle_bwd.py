"""Pins of the oracle's backward pass (CPU).

The backward oracle is checked against things other than itself:

* central finite differences of the (separately pinned) forward oracle, for
  every gradient, on small random problems covering the gated / ungated,
  softplus on / off, with / without D, bias, initial and final state cases;
* the adjoint identity <dL/dx, v> = d/de L(x + e v) for a random direction v
  in all inputs at once;
* closed forms: dD = sum_t dy SiLU(z) u; with dy = 0 and dL/d(final state)
  given, d(initial state) = exp(A sum_t Delta_t) dL/d(final state) and every
  readout-side gradient is zero; with C = 0 and D = 0 the output is zero and
  so are dz, du and ddelta;
* planted mistakes in copies of the backward code, each of which must fail
  one of the pins above;
* the same finite-difference pins for the Euler input term, with planted
  mistakes in its branch.
"""
import numpy as np
import pytest

import oracle

NAMES = [("u", "du"), ("delta", "ddelta"), ("A_log", "dA_log"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
         ("z", "dz"), ("delta_bias", "ddelta_bias"), ("initial_state", "d_initial_state")]


def problem(b, d, n, L, gated=True, hasD=True, hasbias=True, h0=True, dfs=True, seed=0):
    rng = np.random.default_rng(seed)
    p = dict(u=rng.standard_normal((b, d, L)), delta=rng.standard_normal((b, d, L)),
             A_log=np.log(rng.uniform(0.5, 3.0, (d, n))), B=rng.standard_normal((b, n, L)),
             C=rng.standard_normal((b, n, L)),
             D=rng.standard_normal(d) if hasD else None,
             z=rng.standard_normal((b, d, L)) if gated else None,
             delta_bias=rng.uniform(-2.0, 0.5, d) if hasbias else None,
             initial_state=rng.standard_normal((b, d, n)) * 0.3 if h0 else None)
    dy = rng.standard_normal((b, d, L))
    dfs_ = rng.standard_normal((b, d, n)) if dfs else None
    return p, dy, dfs_


def loss(o, p, dy, dfs, softplus, disc="zoh"):
    y, fs = o.scan_fwd(**p, delta_softplus=softplus, discretization=disc)
    out = float((y * dy).sum())
    if dfs is not None:
        out += float((fs * dfs).sum())
    return out


def fd_grads(o, p, dy, dfs, softplus, eps=1e-6, disc="zoh"):
    g = {}
    for name, key in NAMES:
        arr = p[name]
        if arr is None:
            continue
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            pp = dict(p)
            a1 = arr.copy()
            a1[idx] += eps
            pp[name] = a1
            lp = loss(o, pp, dy, dfs, softplus, disc)
            a2 = arr.copy()
            a2[idx] -= eps
            pp[name] = a2
            lm = loss(o, pp, dy, dfs, softplus, disc)
            fd[idx] = (lp - lm) / (2 * eps)
        g[key] = fd
    return g


def bwd(o, p, dy, dfs, softplus, disc="zoh"):
    return o.scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], dy, D=p["D"], z=p["z"],
                      delta_bias=p["delta_bias"], initial_state=p["initial_state"], d_final_state=dfs,
                      delta_softplus=softplus, discretization=disc)


def check_fd(o, p, dy, dfs, softplus, tol=1e-7, disc="zoh"):
    g = bwd(o, p, dy, dfs, softplus, disc)
    ref = fd_grads(o, p, dy, dfs, softplus, disc=disc)
    for key, fd in ref.items():
        err = np.abs(g[key] - fd).max() / max(np.abs(fd).max(), 1e-12)
        assert err < tol, (key, err)


CASES = [
    # (b, d, n, L, gated, hasD, hasbias, h0, dfs, softplus)
    (2, 3, 4, 9, True, True, True, True, True, True),
    (1, 2, 1, 1, True, True, True, True, True, True),
    (2, 2, 5, 7, False, False, False, False, False, True),
    (1, 3, 16, 13, True, True, True, False, True, False),
    (2, 1, 3, 6, False, True, False, True, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}" + ("g" if c[4] else "")
                                            + ("" if c[9] else "-nosp") for c in CASES])
def test_bwd_matches_finite_differences(case):
    b, d, n, L, gated, hasD, hasbias, h0, dfs, sp = case
    p, dy, dfs_ = problem(b, d, n, L, gated, hasD, hasbias, h0, dfs, seed=L + 10 * n)
    if not sp:
        p["delta"] = np.abs(p["delta"]) * 0.5 + 0.01   # a positive step without softplus
        p["delta_bias"] = None if p["delta_bias"] is None else np.abs(p["delta_bias"]) * 0.1
    check_fd(oracle, p, dy, dfs_, sp)


@pytest.mark.parametrize("case", CASES[:4], ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}" + ("g" if c[4] else "")
                                                + ("" if c[9] else "-nosp") for c in CASES[:4]])
def test_bwd_euler_matches_finite_differences(case):
    """The Euler input term (Bbar u = Delta B u): every gradient against finite differences of the
    Euler forward oracle (itself pinned to the zero-order hold to O(Delta^2))."""
    b, d, n, L, gated, hasD, hasbias, h0, dfs, sp = case
    p, dy, dfs_ = problem(b, d, n, L, gated, hasD, hasbias, h0, dfs, seed=L + 10 * n + 1)
    if not sp:
        p["delta"] = np.abs(p["delta"]) * 0.5 + 0.01
        p["delta_bias"] = None if p["delta_bias"] is None else np.abs(p["delta_bias"]) * 0.1
    check_fd(oracle, p, dy, dfs_, sp, disc="euler")


def test_bwd_euler_differs_from_zoh():
    p, dy, dfs = problem(2, 3, 4, 9, seed=12)
    ge, gz = bwd(oracle, p, dy, dfs, True, "euler"), bwd(oracle, p, dy, dfs, True, "zoh")
    for k in ("du", "ddelta", "dA_log", "dB", "dz"):
        assert np.abs(ge[k] - gz[k]).max() > 1e-6, k


def test_bwd_adjoint_identity():
    p, dy, dfs = problem(3, 4, 8, 20, seed=5)
    rng = np.random.default_rng(6)
    v = {k: (None if a is None else rng.standard_normal(a.shape)) for k, a in p.items()}
    g = bwd(oracle, p, dy, dfs, True)
    lhs = sum(float((g[key] * v[name]).sum()) for name, key in NAMES)
    eps = 1e-6
    pp = {k: (None if a is None else a + eps * v[k]) for k, a in p.items()}
    pm = {k: (None if a is None else a - eps * v[k]) for k, a in p.items()}
    rhs = (loss(oracle, pp, dy, dfs, True) - loss(oracle, pm, dy, dfs, True)) / (2 * eps)
    assert abs(lhs - rhs) <= 1e-7 * max(1.0, abs(rhs))


def test_bwd_dD_closed_form():
    p, dy, dfs = problem(2, 3, 4, 11, seed=7)
    g = bwd(oracle, p, dy, dfs, True)
    z = p["z"]
    silu = z / (1.0 + np.exp(-z))
    np.testing.assert_allclose(g["dD"], (dy * silu * p["u"]).sum(axis=(0, 2)), rtol=1e-12, atol=1e-12)


def test_bwd_final_state_only():
    """dy = 0: only the final state carries gradient; it decays back through the
    whole sequence to exp(A sum Delta) dL/d(final state)."""
    p, dy, dfs = problem(2, 3, 5, 10, seed=8)
    dy = np.zeros_like(dy)
    g = bwd(oracle, p, dy, dfs, True)
    A = -np.exp(p["A_log"])
    x = p["delta"] + p["delta_bias"][None, :, None]
    Delta = np.logaddexp(0.0, x)                                  # softplus
    decay = np.exp(A[None, :, :] * Delta.sum(axis=2)[:, :, None])
    np.testing.assert_allclose(g["d_initial_state"], decay * dfs, rtol=1e-12, atol=1e-14)
    assert np.all(g["dC"] == 0) and np.all(g["dz"] == 0) and np.all(g["dD"] == 0)


def test_bwd_zero_readout():
    """C = 0 and D = 0: the output is identically zero, so dz, du and ddelta vanish."""
    p, dy, _ = problem(2, 3, 4, 9, seed=9)
    p["C"] = np.zeros_like(p["C"])
    p["D"] = np.zeros_like(p["D"])
    g = bwd(oracle, p, dy, None, True)
    for k in ("dz", "du", "ddelta", "dB", "dA_log", "ddelta_bias", "d_initial_state"):
        assert np.all(g[k] == 0), k


BWD_MUTANTS = [
    ("dDelta_sign", "dDelta += l * Abar * (A[n] * hprev + Bn * ut);",
     "dDelta += l * Abar * (-A[n] * hprev + Bn * ut);"),
    ("lam_no_decay", "lam[n] = Abar * l;", "lam[n] = l;"),
    ("dB_euler", "pB[n * L + t] += l * ut * bq;", "pB[n * L + t] += l * ut * Delta;"),
    ("silu_derivative", "dz[row + t] = dyt * yt[t] * sg * (1.0 + zz * (1.0 - sg));",
     "dz[row + t] = dyt * yt[t] * sg;"),
    ("final_state_grad_ignored", "lam[n] = d_final_state ? d_final_state[bd * N + n] : 0.0;", "lam[n] = 0.0;"),
    ("dA_log_chain_factor", "dA_log[d * N + n] = pdim[d * (N + 2) + n] * (-exp(A_log[d * N + n]));",
     "dA_log[d * N + n] = pdim[d * (N + 2) + n];"),
    ("dC_old_state", "pC[n * L + t] += dyt * H[(t + 1) * N + n];", "pC[n * L + t] += dyt * H[t * N + n];"),
    ("softplus_grad_no_bias", "dDelta * oracle_sigmoid(delta[row + t] + bias)", "dDelta * oracle_sigmoid(delta[row + t])"),
    ("du_no_bbar", "dut += l * bq * Bn;", "dut += l * Bn;"),
    ("dA_missing_input_term", "dAn[n] += l * (Delta * Abar * hprev + ut * Bn * dbq);",
     "dAn[n] += l * (Delta * Abar * hprev);"),
]
# planted mistakes in the Euler branch, caught by the Euler finite differences
BWD_EULER_MUTANTS = [
    ("euler_dDelta_zoh_form", "dDelta += l * (Abar * A[n] * hprev + Bn * ut);",
     "dDelta += l * Abar * (A[n] * hprev + Bn * ut) + 0.0;"),
    ("euler_bbar_zoh", "const double bq = euler ? Delta : ", "const double bq = euler ? em1 / A[n] : "),
    ("euler_dA_input_term", "const double dbq = euler ? 0.0 : ", "const double dbq = euler ? 0.5 * Delta * Delta : "),
]


@pytest.mark.parametrize("name,old,new", BWD_EULER_MUTANTS, ids=[m[0] for m in BWD_EULER_MUTANTS])
def test_bwd_euler_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, name
    var = oracle.build_variant(src.replace(old, new), str(tmp_path), "me_" + name)
    p, dy, dfs = problem(2, 3, 4, 9, seed=4)
    with pytest.raises(AssertionError):
        check_fd(var, p, dy, dfs, True, disc="euler")


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, name
    var = oracle.build_variant(src.replace(old, new), str(tmp_path), "m_" + name)
    p, dy, dfs = problem(2, 3, 4, 9, seed=3)   # every feature on: gate, D, bias, both states
    with pytest.raises(AssertionError):
        check_fd(var, p, dy, dfs, True)
