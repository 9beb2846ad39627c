"""Pins of the oracle's variable-length batch (sequences packed along time,
each restarting from its own initial state), derived without the oracle's
loop where possible:

* the products form h_t = (prod Abar) h0 + sum_j (prod Abar) Bbar_j u_j written
  out in numpy per sequence, with ZOH Bbar by expm1 (State space models and
  Mamba, §2), at random inputs with gate, D, bias and initial states;
* equality with the (separately pinned) fixed-length scan run on each
  sequence padded into a batch;
* empty sequences return their initial state; nothing leaks across a boundary
  (changing one sequence's inputs leaves the others' outputs bit-identical);
* planted mistakes (the initial state of the wrong sequence, an off-by-one boundary, a
  wrong B row stride) are caught.
"""
import numpy as np
import pytest

import oracle


def _case(dim, n, lens, rng):
    total = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(u=rng.standard_normal((dim, total)), delta=rng.standard_normal((dim, total)) * 0.7 - 0.5,
                A_log=rng.uniform(-1.0, 1.5, size=(dim, n)), B=rng.standard_normal((n, total)),
                C=rng.standard_normal((n, total)), cu_seqlens=cu, D=rng.standard_normal(dim),
                z=rng.standard_normal((dim, total)), delta_bias=rng.uniform(-1.0, 0.5, size=dim),
                initial_states=rng.standard_normal((len(lens), dim, n)) * 0.3)


def _products(c):
    dim, total = c["u"].shape
    n = c["A_log"].shape[1]
    cu = c["cu_seqlens"]
    Delta = np.logaddexp(0.0, c["delta"] + c["delta_bias"][:, None])
    A = -np.exp(c["A_log"])
    y = np.zeros((dim, total))
    fs = np.zeros((len(cu) - 1, dim, n))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for d in range(dim):
            h0 = c["initial_states"][s, d]
            logA = Delta[d, a:b, None] * A[d][None, :]
            cum = np.concatenate([np.zeros((1, n)), np.cumsum(logA, axis=0)])
            h = h0
            for i, t in enumerate(range(a, b)):
                h = np.exp(cum[i + 1]) * h0
                for j in range(i + 1):
                    tj = a + j
                    bbar = np.expm1(Delta[d, tj] * A[d]) / A[d] * c["B"][:, tj]
                    h = h + np.exp(cum[i + 1] - cum[j + 1]) * bbar * c["u"][d, tj]
                yt = np.dot(c["C"][:, t], h) + c["D"][d] * c["u"][d, t]
                zt = c["z"][d, t]
                y[d, t] = yt * zt / (1 + np.exp(-zt))
            fs[s, d] = h
    return y, fs


@pytest.mark.parametrize("lens", [(3, 0, 5, 1), (7,), (0, 0, 4)])
def test_varlen_products_form(lens, o=oracle):
    c = _case(3, 4, lens, np.random.default_rng(sum(lens) + len(lens)))
    y, fs = o.scan_fwd_varlen(**c)
    yr, fr = _products(c)
    np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(fs, fr, rtol=1e-10, atol=1e-12)


def test_varlen_equals_padded_batch(o=oracle):
    lens = (9, 1, 0, 14, 6)
    c = _case(5, 6, lens, np.random.default_rng(3))
    y, fs = o.scan_fwd_varlen(**c, discretization="euler")
    cu, L = c["cu_seqlens"], max(lens)
    for s, ln in enumerate(lens):
        if ln == 0:
            assert np.array_equal(fs[s], c["initial_states"][s])
            continue
        sl = slice(cu[s], cu[s + 1])
        yb, fb = oracle.scan_fwd(c["u"][None, :, sl], c["delta"][None, :, sl], c["A_log"], c["B"][None, :, sl],
                                 c["C"][None, :, sl], D=c["D"], z=c["z"][None, :, sl], delta_bias=c["delta_bias"],
                                 initial_state=c["initial_states"][s:s + 1], discretization="euler")
        assert np.array_equal(y[:, sl], yb[0]) and np.array_equal(fs[s], fb[0])


def test_varlen_no_leak_across_boundary(o=oracle):
    lens = (6, 5, 7)
    c = _case(2, 3, lens, np.random.default_rng(11))
    y, fs = o.scan_fwd_varlen(**c)
    c2 = dict(c)
    c2["u"] = c["u"].copy()
    c2["u"][:, 6:11] += 1.0            # only the second sequence changes
    y2, fs2 = o.scan_fwd_varlen(**c2)
    assert np.array_equal(y2[:, :6], y[:, :6]) and np.array_equal(y2[:, 11:], y[:, 11:])
    assert np.array_equal(fs2[0], fs[0]) and np.array_equal(fs2[2], fs[2])
    assert not np.array_equal(y2[:, 6:11], y[:, 6:11])


def test_varlen_rejects_bad_offsets():
    c = _case(1, 1, (2, 2), np.random.default_rng(1))
    c["cu_seqlens"] = np.array([0, 3, 2], dtype=np.int64)
    with pytest.raises(ValueError):
        oracle.scan_fwd_varlen(**c)


VARLEN_MUTANTS = [
    ("initial_state_of_wrong_sequence", "h[n] = initial_states ? initial_states[sd * dstate + n] : 0.0;   /* restart at the sequence start */",
     "h[n] = initial_states ? initial_states[d * dstate + n] : 0.0;"),
    ("boundary_off_by_one", "for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {",
     "for (int64_t t = cu_seqlens[s] + (s > 0); t < cu_seqlens[s + 1]; ++t) {"),
    ("B_row_stride", "B + t, total, C + t, total, Dd", "B + t, total - 1, C + t, total, Dd"),
]

VARLEN_PINS = [
    lambda o: test_varlen_products_form((3, 0, 5, 1), o),
    test_varlen_no_leak_across_boundary,
]


@pytest.mark.parametrize("name,old,new", VARLEN_MUTANTS, ids=[m[0] for m in VARLEN_MUTANTS])
def test_varlen_planted_mistake_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert old in src, f"mutation site for {name} not found"
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path), "mut_" + name)
    caught = 0
    for pin in VARLEN_PINS:
        try:
            pin(variant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught, f"no pin caught the planted mistake {name}"
