"""Pins of the oracle's multi-head SSM with a scalar decay per head (the
state-space-duality form; State space models and Mamba, §5), each derived
without the oracle's loop:

* reduction to the (separately pinned) selective-scan oracle: with A and
  Delta shared by the P channels of a head and B, C shared by all heads, the
  two are the same function;
* the dual (semiseparable) matrix form y = M x with
  M_ij = (C_i . B_j) Lambda_ij w_j, Lambda_ij = prod_{t=j+1..i} a_t, built with
  numpy from cumulative sums of log a (plus the decayed initial state);
* the chunked algorithm (§5: Q x Q matrix products inside a chunk, only the
  N x P state passed between chunks) in numpy, for chunk sizes 1, 3, 8 and L;
* planted mistakes in copies of the oracle are caught.
"""
import numpy as np
import pytest

import oracle


def _case(b, L, H, P, N, rng, gated=True, h0=True):
    return dict(x=rng.standard_normal((b, L, H, P)), dt=rng.standard_normal((b, L, H)) * 0.7 - 0.5,
                A_log=rng.uniform(-1.0, 1.0, size=H), B=rng.standard_normal((b, L, N)),
                C=rng.standard_normal((b, L, N)), D=rng.standard_normal(H),
                z=rng.standard_normal((b, L, H, P)) if gated else None, dt_bias=rng.uniform(-1.0, 0.5, size=H),
                initial_state=rng.standard_normal((b, H, P, N)) * 0.3 if h0 else None)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _terms(c, disc):
    Delta = np.logaddexp(0.0, c["dt"] + c["dt_bias"][None, None, :])      # (b, L, H)
    A = -np.exp(c["A_log"])                                                 # (H,)
    loga = Delta * A[None, None, :]
    w = Delta if disc == "euler" else np.expm1(loga) / A[None, None, :]
    return loga, w


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_ssd_reduces_to_selective_scan(disc):
    b, L, H, P, N = 2, 11, 3, 4, 5
    c = _case(b, L, H, P, N, np.random.default_rng(1))
    y, fs = oracle.ssd_fwd(**c, discretization=disc)
    dim = H * P
    u = c["x"].reshape(b, L, dim).transpose(0, 2, 1)
    delta = np.repeat(c["dt"], P, axis=2).transpose(0, 2, 1)            # head h -> channels h*P .. h*P+P-1
    A_log = np.repeat(c["A_log"], P)[:, None] * np.ones((1, N))
    y1, f1 = oracle.scan_fwd(u, delta, A_log, c["B"].transpose(0, 2, 1), c["C"].transpose(0, 2, 1),
                             D=np.repeat(c["D"], P), z=c["z"].reshape(b, L, dim).transpose(0, 2, 1),
                             delta_bias=np.repeat(c["dt_bias"], P), initial_state=c["initial_state"].reshape(b, dim, N),
                             discretization=disc)
    np.testing.assert_allclose(y.reshape(b, L, dim).transpose(0, 2, 1), y1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fs.reshape(b, dim, N), f1, rtol=1e-12, atol=1e-12)


def _dual_form(c, disc):
    loga, w = _terms(c, disc)
    b_, L, H, P = c["x"].shape
    y = np.zeros_like(c["x"])
    for b in range(b_):
        for h in range(H):
            cs = np.concatenate([[0.0], np.cumsum(loga[b, :, h])])           # cs[i+1] = sum_{t<=i} log a_t
            seg = cs[1:, None] - cs[None, 1:]                                 # sum_{t=j+1..i} log a_t
            lam = np.where(np.tril(np.ones((L, L))) > 0, np.exp(np.where(seg <= 0, seg, 0.0)), 0.0)
            M = (c["C"][b] @ c["B"][b].T) * lam * w[b, :, h][None, :]
            yh = M @ c["x"][b, :, h, :]                                       # (L, P)
            if c["initial_state"] is not None:
                yh += np.exp(cs[1:])[:, None] * (c["C"][b] @ c["initial_state"][b, h].T)
            yh += c["D"][h] * c["x"][b, :, h, :]
            if c["z"] is not None:
                yh *= _silu(c["z"][b, :, h, :])
            y[b, :, h, :] = yh
    return y


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_ssd_dual_matrix_form(disc):
    c = _case(2, 13, 2, 3, 4, np.random.default_rng(2))
    y, _ = oracle.ssd_fwd(**c, discretization=disc)
    np.testing.assert_allclose(y, _dual_form(c, disc), rtol=1e-10, atol=1e-12)


def _chunked(c, Q, disc):
    """Chunk-wise algorithm: per chunk, y = (G o Lmask o w) x + diag(exp(cum)) C S_in + D x and
    S_out = exp(cum_end) S_in + B^T diag(exp(cum_end - cum_j) w_j) x."""
    loga, w = _terms(c, disc)
    b_, L, H, P = c["x"].shape
    N = c["B"].shape[-1]
    y = np.zeros_like(c["x"])
    fs = np.zeros((b_, H, P, N))
    for b in range(b_):
        for h in range(H):
            S = (c["initial_state"][b, h].T.copy() if c["initial_state"] is not None else np.zeros((N, P)))
            for t0 in range(0, L, Q):
                t1 = min(L, t0 + Q)
                la = loga[b, t0:t1, h]
                cum = np.cumsum(la)
                Cc, Bc, Xc = c["C"][b, t0:t1], c["B"][b, t0:t1], c["x"][b, t0:t1, h, :]
                seg = cum[:, None] - cum[None, :]
                Lm = np.where(np.tril(np.ones((t1 - t0, t1 - t0))) > 0, np.exp(np.minimum(seg, 0.0)), 0.0)
                Mc = (Cc @ Bc.T) * Lm * w[b, t0:t1, h][None, :]
                yc = Mc @ Xc + np.exp(cum)[:, None] * (Cc @ S) + c["D"][h] * Xc
                if c["z"] is not None:
                    yc *= _silu(c["z"][b, t0:t1, h, :])
                y[b, t0:t1, h, :] = yc
                S = np.exp(cum[-1]) * S + Bc.T @ (np.exp(cum[-1] - cum)[:, None] * w[b, t0:t1, h][:, None] * Xc)
            fs[b, h] = S.T
    return y, fs


@pytest.mark.parametrize("Q", [1, 3, 8, 19])
def test_ssd_chunked_algorithm(Q):
    c = _case(1, 19, 2, 3, 5, np.random.default_rng(3 + Q))
    y, fs = oracle.ssd_fwd(**c)
    yc, fc = _chunked(c, Q, "zoh")
    np.testing.assert_allclose(y, yc, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fs, fc, rtol=1e-10, atol=1e-12)


def test_ssd_empty_sequence_keeps_state():
    c = _case(1, 0, 2, 3, 4, np.random.default_rng(4))
    y, fs = oracle.ssd_fwd(**c)
    assert y.shape == (1, 0, 2, 3)
    assert np.array_equal(fs, c["initial_state"])


SSD_MUTANTS = [
    ("decay_of_wrong_head", "const double A = -exp(A_log[hh]);", "const double A = -exp(A_log[p % nheads]);"),
    ("input_weight_dropped", "h[n] = a * h[n] + w * Bt[n] * x[xi];", "h[n] = a * h[n] + Bt[n] * x[xi];"),
    ("B_reads_C", "const double* Bt = B + (b * seqlen + t) * dstate;", "const double* Bt = C + (b * seqlen + t) * dstate;"),
    ("D_dropped", "double yv = acc + Dh * x[xi];", "double yv = acc;"),
    ("dt_of_wrong_head", "const double xv = dt[(b * seqlen + t) * nheads + hh] + bias;",
     "const double xv = dt[(b * seqlen + t) * nheads] + bias;"),
    ("state_transposed", "h[n] = initial_state ? initial_state[((b * nheads + hh) * headdim + p) * dstate + n] : 0.0;",
     "h[n] = initial_state ? initial_state[((b * nheads + hh) * dstate + n) * headdim + p] : 0.0;"),
]

SSD_PINS = [
    lambda o: _pin_reduction(o),
    lambda o: _pin_dual(o),
]


def _pin_reduction(o):
    b, L, H, P, N = 1, 6, 2, 3, 4
    c = _case(b, L, H, P, N, np.random.default_rng(5))
    y, _ = o.ssd_fwd(**c)
    dim = H * P
    y1, _ = oracle.scan_fwd(c["x"].reshape(b, L, dim).transpose(0, 2, 1),
                            np.repeat(c["dt"], P, axis=2).transpose(0, 2, 1),
                            np.repeat(c["A_log"], P)[:, None] * np.ones((1, N)), c["B"].transpose(0, 2, 1),
                            c["C"].transpose(0, 2, 1), D=np.repeat(c["D"], P),
                            z=c["z"].reshape(b, L, dim).transpose(0, 2, 1), delta_bias=np.repeat(c["dt_bias"], P),
                            initial_state=c["initial_state"].reshape(b, dim, N))
    np.testing.assert_allclose(y.reshape(b, L, dim).transpose(0, 2, 1), y1, rtol=1e-10, atol=1e-12)


def _pin_dual(o):
    c = _case(1, 7, 2, 2, 3, np.random.default_rng(6))
    y, _ = o.ssd_fwd(**c)
    np.testing.assert_allclose(y, _dual_form(c, "zoh"), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("name,old,new", SSD_MUTANTS, ids=[m[0] for m in SSD_MUTANTS])
def test_ssd_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert old in src, f"mutation site for {name} not found"
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path), "mut_" + name)
    caught = 0
    for pin in SSD_PINS:
        try:
            pin(variant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught, f"no pin caught the planted mistake {name}"
