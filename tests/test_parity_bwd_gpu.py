"""Backward pass on the GPU (through the C ABI) against the fp64 oracle.

Every gradient is compared element by element with the error metric of the
forward tests (max |g - r| / max(|r|, rms(r))) at the io dtype's tolerance
(d_state up to 64, zero-order hold and Euler):
1e-4 for float32 io, 1e-2 for bfloat16 io (gradients stored in bf16 are
rounded to nearest even).  Shapes span several 64-channel workgroups, several
32-token tiles and ragged tails in both; the 130M-layer shape is compared in
full.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_55_amd as mscan
from workloads import backward_inputs, by_name, err_report, forward_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
KEYS = ["du", "ddelta", "dA_log", "dB", "dC", "dD", "dz", "ddelta_bias", "d_initial_state"]


def say(msg):
    print(f"[bwd] {msg}", flush=True)


def dev(t):
    return None if t is None else t.to("cuda:0")


def grad_inputs(inp, seed, with_dfs):
    b, d, L = inp["u"].shape
    io = "bf16" if inp["u"].dtype == torch.bfloat16 else "f32"
    return backward_inputs(b, d, inp["A_log"].shape[1], L, io, seed=seed, d_final_state=with_dfs)


def run(inp, dy, dfs, softplus=True, disc="zoh"):
    return mscan.scan_bwd(dev(inp["u"]), dev(inp["delta"]), dev(inp["A_log"]), dev(inp["B"]), dev(inp["C"]),
                          dev(dy), D=dev(inp["D"]), z=dev(inp["z"]), delta_bias=dev(inp["delta_bias"]),
                          initial_state=dev(inp["initial_state"]), d_final_state=dev(dfs),
                          delta_softplus=softplus, discretization=disc)


def ref(inp, dy, dfs, softplus=True, disc="zoh"):
    return oracle.scan_bwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], dy, D=inp["D"], z=inp["z"],
                           delta_bias=inp["delta_bias"], initial_state=inp["initial_state"], d_final_state=dfs,
                           delta_softplus=softplus, discretization=disc)


def check_all(got, want, tol):
    for k in KEYS:
        if want.get(k) is None:
            assert got.get(k) is None, k
            continue
        rep = err_report(got[k].float().cpu(), want[k])
        say(f"  {k}: {rep}")
        assert rep["max_rel"] <= tol, (k, rep)


# (batch, dim, dstate, L, io, gated, has_D, has_bias, h0, dfs, softplus)
CASES = [
    (1, 64, 16, 64, "f32", True, True, True, False, False, True),
    (2, 70, 16, 100, "f32", True, True, True, True, True, True),
    (1, 130, 5, 33, "bf16", True, True, True, True, False, True),
    (2, 64, 16, 1, "f32", True, False, True, True, True, True),
    (1, 3, 1, 31, "f32", False, True, False, False, True, True),
    (2, 192, 16, 257, "bf16", True, True, True, True, True, True),
    (1, 128, 8, 96, "f32", False, False, False, True, False, False),
    (3, 65, 12, 160, "bf16", False, True, True, False, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}{c[4]}" + ("g" if c[5] else "")
                                            + ("" if c[10] else "-nosp") for c in CASES])
def test_bwd_vs_oracle(case):
    b, d, n, L, io, gated, hasD, hasB, h0, dfs_on, sp = case
    inp = forward_inputs(batch=b, dim=d, dstate=n, seqlen=L, io=io, gated=gated, has_D=hasD, has_bias=hasB,
                         initial_state=h0, seed=L + d)
    if not sp:
        inp["delta"] = (inp["delta"].float().abs() * 0.05).to(inp["delta"].dtype)
    dy, dfs = grad_inputs(inp, seed=L * 7 + d, with_dfs=dfs_on)
    say(f"case {case}")
    got = run(inp, dy, dfs, sp)
    want = ref(inp, dy, dfs, sp)
    check_all(got, want, TOL[io])


@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[5], CASES[6]],
                         ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}{c[4]}" + ("g" if c[5] else "") + ("" if c[10] else "-nosp")
                              for c in [CASES[1], CASES[2], CASES[5], CASES[6]]])
def test_bwd_euler_vs_oracle(case):
    """The Euler input term (Bbar u = Delta B u): every gradient against the oracle."""
    b, d, n, L, io, gated, hasD, hasB, h0, dfs, sp = case
    inp = forward_inputs(batch=b, dim=d, dstate=n, seqlen=L, io=io, gated=gated, has_D=hasD, has_bias=hasB,
                         initial_state=h0, seed=L + d + 1)
    if not sp:
        inp["delta"] = (inp["delta"].float().abs() * 0.05).to(inp["delta"].dtype)
    dy, dfs_t = grad_inputs(inp, seed=L + 1, with_dfs=dfs)
    say(f"euler case {case}")
    got = run(inp, dy, dfs_t, sp, "euler")
    want = ref(inp, dy, dfs_t, sp, "euler")
    check_all(got, want, TOL[io])


WIDE = [  # d_state above 16: one checkpoint + gradient pass per 16 states
    (2, 70, 32, 100, "f32", True, True, True, True, True, True),
    (1, 130, 64, 33, "bf16", True, True, True, True, False, True),
    (2, 64, 20, 257, "bf16", False, True, False, False, True, True),
    (1, 96, 48, 96, "f32", True, False, False, True, True, False),   # no softplus: no bias, so Delta > 0
]


@pytest.mark.parametrize("case", WIDE, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}{c[4]}" + ("g" if c[5] else "")
                                            + ("" if c[10] else "-nosp") for c in WIDE])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_wide_state_vs_oracle(case, disc):
    b, d, n, L, io, gated, hasD, hasB, h0, dfs_on, sp = case
    inp = forward_inputs(batch=b, dim=d, dstate=n, seqlen=L, io=io, gated=gated, has_D=hasD, has_bias=hasB,
                         initial_state=h0, seed=L + d + n)
    if not sp:
        inp["delta"] = (inp["delta"].float().abs() * 0.05).to(inp["delta"].dtype)
    dy, dfs = grad_inputs(inp, seed=L * 3 + n, with_dfs=dfs_on)
    say(f"wide case {case} {disc}")
    got = run(inp, dy, dfs, sp, disc)
    want = ref(inp, dy, dfs, sp, disc)
    check_all(got, want, TOL[io])


def test_bwd_deterministic():
    inp = forward_inputs(batch=2, dim=256, dstate=16, seqlen=300, io="bf16", initial_state=True, seed=3)
    dy, dfs = grad_inputs(inp, seed=4, with_dfs=True)
    say("determinism")
    g1 = run(inp, dy, dfs)
    g2 = run(inp, dy, dfs)
    for k in KEYS:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_bwd_seqlen_zero():
    inp = forward_inputs(batch=2, dim=70, dstate=16, seqlen=0, io="bf16", initial_state=True, seed=1)
    dy, dfs = backward_inputs(2, 70, 16, 0, "bf16", seed=1, d_final_state=True)
    say("seqlen 0")
    g = run(inp, dy, dfs)
    assert torch.equal(g["d_initial_state"].cpu(), dfs)
    assert torch.all(g["dA_log"] == 0) and torch.all(g["dD"] == 0) and torch.all(g["ddelta_bias"] == 0)


def test_bwd_config1_full():
    """The 130M-layer shape (b8 d1536 L2048, bf16, gated), every gradient in full."""
    c = by_name("mamba-130m-layer")
    inp = forward_inputs(c)
    dy, _ = grad_inputs(inp, seed=11, with_dfs=False)
    say("mamba-130m-layer full backward")
    got = run(inp, dy, None)
    want = ref(inp, dy, None)
    check_all(got, want, c.tol)
