"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each check below derives the expected result by a route that shares nothing
with the oracle's sequential loop:

* ZOH by the matrix exponential of the augmented continuous system (Van Loan's
  block identity; scipy.linalg.expm), products of Abar written out, and the
  semiseparable matrix form (State space models and Mamba, §2, §5);
* the LTI case as a convolution computed directly and by numpy.fft
  (State space models and Mamba, §3);
* Theorem 1 against scipy.special.expit (State space models and Mamba, §4);
* split/resume and the associative (a, b) fold (State space models and Mamba,
  Parallel Scan; MAMBA walkthrough §2.2, chunked scan);
* chained single-token steps against the full scan (recurrence mode, §3);
* the D skip, the gate (torch.nn.functional.silu) and linearity in u.
"""
import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

RNG = np.random.default_rng(12345)


def _rand_case(b, d, n, L, rng, softplus=True, gated=True, h0=True):
    u = rng.standard_normal((b, d, L))
    # with softplus off, Delta = delta + bias is drawn positive (a step size)
    dl = rng.standard_normal((b, d, L)) * 0.7 - 0.5 if softplus else np.abs(rng.standard_normal((b, d, L))) * 0.5
    A_log = rng.uniform(-1.0, 1.5, size=(d, n))
    B = rng.standard_normal((b, n, L))
    C = rng.standard_normal((b, n, L))
    D = rng.standard_normal(d)
    z = rng.standard_normal((b, d, L)) if gated else None
    bias = rng.uniform(-1.0, 0.5, size=d) if softplus else rng.uniform(0.01, 0.2, size=d)
    init = rng.standard_normal((b, d, n)) * 0.3 if h0 else None
    return dict(u=u, delta=dl, A_log=A_log, B=B, C=C, D=D, z=z, delta_bias=bias, initial_state=init,
                delta_softplus=softplus)


def _delta(case):
    x = case["delta"] + case["delta_bias"][None, :, None]
    return np.logaddexp(0.0, x) if case["delta_softplus"] else x   # softplus via numpy.logaddexp


def _zoh_vanloan(A_diag, Bvec, Delta):
    """ZOH of dh/dt = diag(A) h + B u over a step Delta with u held constant:
    expm([[A, B], [0, 0]] * Delta) = [[Abar, Bbar], [0, 1]]."""
    n = len(A_diag)
    M = np.zeros((n + 1, n + 1))
    M[:n, :n] = np.diag(A_diag)
    M[:n, n] = Bvec
    E = scipy.linalg.expm(M * Delta)
    return np.diag(E[:n, :n]).copy(), E[:n, n].copy()


def _bruteforce_products(case):
    """h_t = (prod_{s<=t} Abar_s) h0 + sum_{j<=t} (prod_{s=j+1..t} Abar_s) Bbar_j u_j."""
    u, C = case["u"], case["C"]
    b_, d_, L = u.shape
    n = case["A_log"].shape[1]
    A = -np.exp(case["A_log"])
    Dl = _delta(case)
    y = np.zeros_like(u)
    fs = np.zeros((b_, d_, n))
    for b in range(b_):
        for d in range(d_):
            Abar = np.zeros((L, n))
            Bbar = np.zeros((L, n))
            for t in range(L):
                Abar[t], Bbar[t] = _zoh_vanloan(A[d], case["B"][b, :, t], Dl[b, d, t])
            h0 = case["initial_state"][b, d] if case["initial_state"] is not None else np.zeros(n)
            for t in range(L):
                h = np.prod(Abar[: t + 1], axis=0) * h0
                for j in range(t + 1):
                    h = h + np.prod(Abar[j + 1: t + 1], axis=0) * Bbar[j] * u[b, d, j]
                yt = C[b, :, t] @ h + case["D"][d] * u[b, d, t]
                if case["z"] is not None:
                    zz = case["z"][b, d, t]
                    yt = yt * zz * scipy.special.expit(zz)
                y[b, d, t] = yt
                if t == L - 1:
                    fs[b, d] = h
    return y, fs


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("shape", [(1, 1, 1, 5), (2, 3, 4, 8), (1, 2, 16, 6), (2, 1, 3, 7)])
@pytest.mark.parametrize("softplus,gated,h0", [(True, True, True), (False, False, False), (True, False, True)])
def test_products_vanloan(oracle_mod, shape, softplus, gated, h0):
    case = _rand_case(*shape, RNG, softplus=softplus, gated=gated, h0=h0)
    y, fs = oracle_mod.scan_fwd(**case)
    yr, fsr = _bruteforce_products(case)
    assert _rel(y, yr) < 1e-12
    assert _rel(fs, fsr) < 1e-12


def test_semiseparable_matrix(oracle_mod):
    """Y = M U with M[i,j] = sum_n C_i[n] (prod_{s=j+1..i} Abar_s[n]) Bbar_j[n] (lower triangular)."""
    case = _rand_case(1, 3, 16, 40, RNG, gated=True, h0=False)
    y, _ = oracle_mod.scan_fwd(**case)
    A = -np.exp(case["A_log"])
    Dl = _delta(case)
    L = 40
    for d in range(3):
        Abar = np.zeros((L, 16))
        Bbar = np.zeros((L, 16))
        for t in range(L):
            Abar[t], Bbar[t] = _zoh_vanloan(A[d], case["B"][0, :, t], Dl[0, d, t])
        M = np.zeros((L, L))
        for i in range(L):
            for j in range(i + 1):
                lam = np.prod(Abar[j + 1: i + 1], axis=0)
                M[i, j] = np.sum(case["C"][0, :, i] * lam * Bbar[j])
        # rank of every strictly-lower block is at most N (semiseparable); a sanity property
        assert np.linalg.matrix_rank(M[20:, :20], tol=1e-10) <= 16
        yy = M @ case["u"][0, d] + case["D"][d] * case["u"][0, d]
        zz = case["z"][0, d]
        yy = yy * zz * scipy.special.expit(zz)
        assert _rel(y[0, d], yy) < 1e-12


@pytest.mark.parametrize("L", [1, 17, 256])
def test_lti_convolution_fft(oracle_mod, L):
    """Constant Delta, B, C over time: y = K * u + D u, K_i = sum_n C[n] Abar[n]^i Bbar[n]."""
    rng = np.random.default_rng(L)
    n, d = 16, 2
    A_log = rng.uniform(-1.0, 1.5, (d, n))
    A = -np.exp(A_log)
    dconst = rng.uniform(0.01, 0.3, d)
    Bv = rng.standard_normal(n)
    Cv = rng.standard_normal(n)
    D = rng.standard_normal(d)
    u = rng.standard_normal((1, d, L))
    y, _ = oracle_mod.scan_fwd(u, np.broadcast_to(dconst[None, :, None], (1, d, L)), A_log,
                               np.broadcast_to(Bv[None, :, None], (1, n, L)),
                               np.broadcast_to(Cv[None, :, None], (1, n, L)), D=D, delta_softplus=False)
    for ch in range(d):
        Abar, Bbar = _zoh_vanloan(A[ch], Bv, dconst[ch])
        i = np.arange(L)
        K = (Cv[None, :] * np.exp(np.outer(i, np.log(Abar))) * Bbar[None, :]).sum(axis=1)  # Abar^i
        direct = np.array([np.sum(K[: k + 1][::-1] * u[0, ch, : k + 1]) for k in range(L)])
        nfft = 2 * L
        conv = np.fft.irfft(np.fft.rfft(K, nfft) * np.fft.rfft(u[0, ch], nfft), nfft)[:L]
        assert _rel(direct, conv) < 1e-10
        assert _rel(y[0, ch], direct + D[ch] * u[0, ch]) < 1e-12


@pytest.mark.parametrize("nstates", [1, 16])
def test_theorem1_vs_expit(oracle_mod, nstates):
    """N identical states with A=-1, B=1, C=1/N: h_t = (1 - s_t) h_{t-1} + s_t u_t, s_t = expit(delta_t + bias)."""
    rng = np.random.default_rng(7)
    L = 300
    x = rng.standard_normal(L) * 4.0
    bias = 0.37
    u = rng.standard_normal(L)
    y, fs = oracle_mod.scan_fwd(u.reshape(1, 1, L), (x - bias).reshape(1, 1, L), np.zeros((1, nstates)),
                                np.ones((1, nstates, L)), np.full((1, nstates, L), 1.0 / nstates),
                                delta_bias=np.array([bias]))
    g = scipy.special.expit(x)
    h = 0.0
    ref = np.empty(L)
    for t in range(L):
        h = (1.0 - g[t]) * h + g[t] * u[t]
        ref[t] = h
    assert _rel(y.ravel(), ref) < 1e-13
    assert np.allclose(fs.ravel(), ref[-1], rtol=1e-13, atol=0)


def test_large_delta_reset_random(oracle_mod):
    """Delta = 50: h_t = B_t u_t / |A| and y_t = sum_n C_t B_t u_t / |A_n| + D u_t (to e^-50)."""
    rng = np.random.default_rng(3)
    b, d, n, L = 2, 3, 16, 9
    A_log = rng.uniform(0.0, 1.5, (d, n))   # |A| >= 1, so exp(-50 |A|) < 2e-22
    u = rng.standard_normal((b, d, L))
    B = rng.standard_normal((b, n, L))
    C = rng.standard_normal((b, n, L))
    D = rng.standard_normal(d)
    h0 = rng.standard_normal((b, d, n))
    y, fs = oracle_mod.scan_fwd(u, np.full((b, d, L), 50.0), A_log, B, C, D=D, initial_state=h0,
                                delta_softplus=False)
    absA = np.exp(A_log)
    ref = np.einsum("bnt,bnt,dn,bdt->bdt", C, B, 1.0 / absA, u) + D[None, :, None] * u
    assert _rel(y, ref) < 1e-14
    assert _rel(fs, B[:, None, :, -1] * u[:, :, -1:] / absA[None]) < 1e-14


def test_delta_zero_random(oracle_mod):
    rng = np.random.default_rng(4)
    b, d, n, L = 2, 5, 16, 11
    case = _rand_case(b, d, n, L, rng, softplus=False, gated=False, h0=True)
    case["delta"] = np.zeros((b, d, L))
    case["delta_bias"] = np.zeros(d)
    y, fs = oracle_mod.scan_fwd(**case)
    assert np.array_equal(fs, case["initial_state"])
    ref = np.einsum("bnt,bdn->bdt", case["C"], case["initial_state"]) + case["D"][None, :, None] * case["u"]
    assert _rel(y, ref) < 1e-15


@pytest.mark.parametrize("gated", [True, False])
def test_split_resume_every_k(oracle_mod, gated):
    rng = np.random.default_rng(5)
    b, d, n, L = 2, 3, 16, 24
    case = _rand_case(b, d, n, L, rng, gated=gated)
    y, fs = oracle_mod.scan_fwd(**case)
    for k in range(0, L + 1):
        first = {kk: (v[..., :k] if isinstance(v, np.ndarray) and v.ndim == 3 and v.shape[-1] == L else v)
                 for kk, v in case.items()}
        second = {kk: (v[..., k:] if isinstance(v, np.ndarray) and v.ndim == 3 and v.shape[-1] == L else v)
                  for kk, v in case.items()}
        y1, f1 = oracle_mod.scan_fwd(**first)
        second["initial_state"] = f1
        y2, f2 = oracle_mod.scan_fwd(**second)
        assert _rel(np.concatenate([y1, y2], axis=-1), y) < 1e-13
        assert _rel(f2, fs) < 1e-13


def test_associative_segment_fold(oracle_mod):
    """Per segment: (P, h_end) with P = exp(A sum Delta), h_end from a zero state; folding with
    (a1,b1) o (a2,b2) = (a2 a1, a2 b1 + b2) reproduces the final state."""
    rng = np.random.default_rng(6)
    b, d, n, L = 1, 4, 16, 60
    case = _rand_case(b, d, n, L, rng, gated=False)
    _, fs = oracle_mod.scan_fwd(**case)
    A = -np.exp(case["A_log"])
    Dl = _delta(case)
    bounds = [0, 7, 8, 30, 59, 60]
    acc_a = np.ones((b, d, n))
    acc_b = case["initial_state"].copy()
    for s0, s1 in zip(bounds[:-1], bounds[1:]):
        seg = {kk: (v[..., s0:s1] if isinstance(v, np.ndarray) and v.ndim == 3 and v.shape[-1] == L else v)
               for kk, v in case.items()}
        seg["initial_state"] = None
        _, hend = oracle_mod.scan_fwd(**seg)
        P = np.exp(A[None] * Dl[..., s0:s1].sum(axis=-1)[..., None])
        acc_a, acc_b = P * acc_a, P * acc_b + hend
    assert _rel(acc_b, fs) < 1e-12


@pytest.mark.parametrize("softplus,gated", [(True, True), (False, False)])
def test_chained_steps_equal_scan(oracle_mod, softplus, gated):
    rng = np.random.default_rng(8)
    b, d, n, L = 3, 4, 16, 20
    case = _rand_case(b, d, n, L, rng, softplus=softplus, gated=gated)
    y, fs = oracle_mod.scan_fwd(**case)
    st = case["initial_state"].copy()
    for t in range(L):
        yt, st = oracle_mod.scan_step(st, case["u"][..., t], case["delta"][..., t], case["A_log"],
                                      case["B"][..., t], case["C"][..., t], D=case["D"],
                                      z=case["z"][..., t] if gated else None, dt_bias=case["delta_bias"],
                                      dt_softplus=softplus)
        assert np.array_equal(yt, y[..., t])   # the same arithmetic in the same order
    assert np.array_equal(st, fs)


def test_d_skip_alone(oracle_mod):
    rng = np.random.default_rng(9)
    case = _rand_case(2, 3, 16, 13, rng, gated=True)
    case["C"] = np.zeros_like(case["C"])
    y, _ = oracle_mod.scan_fwd(**case)
    zt = torch.from_numpy(case["z"])
    ref = case["D"][None, :, None] * case["u"] * torch.nn.functional.silu(zt).numpy()
    assert _rel(y, ref) < 1e-15


def test_gate_matches_torch_silu(oracle_mod):
    rng = np.random.default_rng(10)
    case = _rand_case(2, 3, 16, 13, rng, gated=True)
    yg, fg = oracle_mod.scan_fwd(**case)
    z = case.pop("z")
    yu, fu = oracle_mod.scan_fwd(z=None, **case)
    ref = yu * torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert _rel(yg, ref) < 1e-14
    assert np.array_equal(fg, fu)
    y0, _ = oracle_mod.scan_fwd(z=np.zeros_like(z), **case)
    assert np.array_equal(y0, np.zeros_like(y0))


def test_linear_in_u(oracle_mod):
    rng = np.random.default_rng(11)
    case = _rand_case(2, 3, 16, 17, rng, gated=False, h0=False)
    u1 = case["u"]
    u2 = rng.standard_normal(u1.shape)
    case.pop("u")
    ya, _ = oracle_mod.scan_fwd(u=1.5 * u1 - 0.25 * u2, **case)
    y1, _ = oracle_mod.scan_fwd(u=u1, **case)
    y2, _ = oracle_mod.scan_fwd(u=u2, **case)
    assert _rel(ya, 1.5 * y1 - 0.25 * y2) < 1e-13


def test_seqlen_zero(oracle_mod):
    rng = np.random.default_rng(12)
    case = _rand_case(2, 3, 4, 0, rng)
    y, fs = oracle_mod.scan_fwd(**case)
    assert y.shape == (2, 3, 0)
    assert np.array_equal(fs, case["initial_state"])
    case["initial_state"] = None
    _, fs0 = oracle_mod.scan_fwd(**case)
    assert np.array_equal(fs0, np.zeros((2, 3, 4)))


def test_nan_propagates(oracle_mod):
    rng = np.random.default_rng(13)
    case = _rand_case(1, 2, 16, 10, rng)
    case["u"][0, 0, 4] = np.nan
    y, fs = oracle_mod.scan_fwd(**case)
    assert np.all(np.isfinite(y[0, 0, :4]))
    assert np.all(np.isnan(y[0, 0, 4:]))
    assert np.all(np.isfinite(y[0, 1]))
    assert np.all(np.isnan(fs[0, 0])) and np.all(np.isfinite(fs[0, 1]))


def test_threads_do_not_change_result(oracle_mod):
    rng = np.random.default_rng(14)
    case = _rand_case(3, 7, 16, 33, rng)
    y1, f1 = oracle_mod.scan_fwd(nthreads=1, **case)
    y8, f8 = oracle_mod.scan_fwd(nthreads=4, **case)
    assert np.array_equal(y1, y8) and np.array_equal(f1, f8)
