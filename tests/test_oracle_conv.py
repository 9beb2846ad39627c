"""Pins of the oracle's causal conv1d + SiLU (CPU): numpy.convolve, torch's SiLU,
the initial-state convention, split/resume bit-exactness, causality, and
planted mistakes in copies of the oracle that must each fail a pin."""
import numpy as np
import pytest
import torch

import oracle


def rand(seed, b, d, L, K):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, d, L)), rng.standard_normal((d, K)), rng.standard_normal(d),
            rng.standard_normal((b, d, K - 1)))


def ref_linear(x, w, bias, state=None):
    """Causal conv by numpy.convolve on [state, x] (state zero if absent), plus bias."""
    b, d, L = x.shape
    K = w.shape[1]
    out = np.empty_like(x)
    for i in range(b):
        for j in range(d):
            pre = state[i, j] if state is not None else np.zeros(K - 1)
            full = np.concatenate([pre, x[i, j]])             # input times -(K-1) .. L-1
            # 'valid' correlation: out[t] = sum_k w[k] full[t + k]
            out[i, j] = np.convolve(full, w[j][::-1], mode="valid") + (bias[j] if bias is not None else 0.0)
    return out


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("L", [1, 2, 5, 64])
def test_conv_matches_numpy(K, L):
    x, w, bias, state = rand(K * 10 + L, 2, 3, L, K)
    for use_state in (False, True):
        st = state if use_state else None
        u = oracle.conv1d_fwd(x, w, bias, conv_state=st, silu=False)
        np.testing.assert_allclose(u, ref_linear(x, w, bias, st), rtol=1e-13, atol=1e-13)
        us = oracle.conv1d_fwd(x, w, bias, conv_state=st, silu=True)
        lin = torch.from_numpy(ref_linear(x, w, bias, st))
        np.testing.assert_allclose(us, torch.nn.functional.silu(lin).numpy(), rtol=1e-12, atol=1e-14)


def test_conv_final_state_and_split_resume():
    x, w, bias, state = rand(3, 2, 4, 37, 4)
    u, fs = oracle.conv1d_fwd(x, w, bias, conv_state=state, return_state=True)
    np.testing.assert_array_equal(fs, x[:, :, -3:])
    for k in (1, 2, 3, 10, 36):
        u1, s1 = oracle.conv1d_fwd(x[:, :, :k], w, bias, conv_state=state, return_state=True)
        u2, s2 = oracle.conv1d_fwd(x[:, :, k:], w, bias, conv_state=s1, return_state=True)
        np.testing.assert_array_equal(np.concatenate([u1, u2], axis=2), u)
        np.testing.assert_array_equal(s2, fs)


def test_conv_short_sequence_state():
    """L < K-1: the final state keeps the older inputs from the initial state."""
    x, w, bias, state = rand(4, 1, 2, 2, 4)
    _, fs = oracle.conv1d_fwd(x, w, bias, conv_state=state, return_state=True)
    np.testing.assert_array_equal(fs, np.concatenate([state[:, :, 2:], x], axis=2))


def test_conv_causal():
    x, w, bias, _ = rand(5, 1, 2, 20, 4)
    u = oracle.conv1d_fwd(x, w, bias)
    x2 = x.copy()
    x2[:, :, 12] += 1.0
    u2 = oracle.conv1d_fwd(x2, w, bias)
    np.testing.assert_array_equal(u[:, :, :12], u2[:, :, :12])
    assert np.all(u[:, :, 12:16] != u2[:, :, 12:16])


CONV_MUTANTS = [
    ("taps_reversed", "acc += w[d * K + k] * xv;", "acc += w[d * K + (K - 1 - k)] * xv;"),
    ("bias_dropped", "double acc = bias ? bias[d] : 0.0;\n      for (int64_t k = 0; k < K; ++k) {",
     "double acc = 0.0;\n      for (int64_t k = 0; k < K; ++k) {"),
    ("silu_is_sigmoid", "u[bd * seqlen + t] = silu_on ? acc * oracle_sigmoid(acc) : acc;",
     "u[bd * seqlen + t] = silu_on ? oracle_sigmoid(acc) : acc;"),
    ("state_off_by_one", "xv = conv_state_in ? conv_state_in[bd * S + (S + tt)] : 0.0;",
     "xv = conv_state_in ? conv_state_in[bd * S + (S + tt - 1 < 0 ? 0 : S + tt - 1)] : 0.0;"),
    ("lookahead", "const int64_t tt = t - S + k;   /* input time of tap k */", "const int64_t tt = t - S + k + 1;"),
]


@pytest.mark.parametrize("name,old,new", CONV_MUTANTS, ids=[m[0] for m in CONV_MUTANTS])
def test_conv_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, name
    var = oracle.build_variant(src.replace(old, new), str(tmp_path), "c_" + name)
    x, w, bias, state = rand(7, 2, 3, 9, 4)
    failed = 0
    for s in (False, True):
        want = ref_linear(x, w, bias, state)
        if s:
            want = torch.nn.functional.silu(torch.from_numpy(want)).numpy()
        try:
            np.testing.assert_allclose(var.conv1d_fwd(x, w, bias, conv_state=state, silu=s), want,
                                       rtol=1e-12, atol=1e-12)
        except AssertionError:
            failed += 1
    assert failed, f"mutant {name} passed"
