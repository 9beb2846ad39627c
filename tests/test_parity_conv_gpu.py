"""Causal conv1d + SiLU on the GPU (through the C ABI) against the fp64 oracle:
K = 1..4, ragged lengths (not multiples of the 8-token thread piece), with and
without bias, SiLU and conv state, fp32 and bf16; split/resume through the
conv state must reproduce the one-shot result bit for bit; the state can be
updated in place."""
import pytest
import torch

import oracle
import selective_state_space_55_amd as mscan
from workloads import conv_inputs, err_report

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(msg):
    print(f"[conv] {msg}", flush=True)


def dev(t):
    return None if t is None else t.to("cuda:0")


CASES = [  # (batch, dim, L, K, io, bias, silu, state)
    (1, 64, 256, 4, "f32", True, True, False),
    (2, 70, 1, 4, "f32", True, True, True),
    (2, 5, 13, 3, "bf16", False, True, True),
    (1, 3, 2, 4, "f32", True, False, True),
    (3, 33, 100, 2, "bf16", True, True, False),
    (1, 8, 31, 1, "f32", True, True, False),
    (2, 130, 2049, 4, "bf16", True, True, True),
    (2, 40, 1536, 4, "f32", True, True, True),
    (1, 16, 1024, 3, "bf16", True, True, True),
    (1, 4, 520, 4, "bf16", True, True, True),
    (1, 6, 1031, 2, "f32", False, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}d{c[1]}L{c[2]}K{c[3]}{c[4]}" for c in CASES])
def test_conv_vs_oracle(case):
    b, d, L, K, io, hb, silu, hs = case
    x, w, bias, st = conv_inputs(b, d, L, K, io, seed=L + K, state=hs)
    bias = bias if hb else None
    say(f"case {case}")
    u, so = mscan.conv1d_fwd(dev(x), dev(w), dev(bias), dev(st), silu=silu, return_state=True)
    ur, sr = oracle.conv1d_fwd(x, w, bias, conv_state=st, silu=silu, return_state=True)
    rep = err_report(u.float().cpu(), ur)
    say(f"  u: {rep}")
    assert rep["max_rel"] <= TOL[io]
    if K > 1:
        assert torch.equal(so.cpu().double(), torch.from_numpy(sr)), "final conv state"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_split_resume_bitexact(io):
    x, w, bias, st = conv_inputs(2, 96, 203, 4, io, seed=9, state=True)
    xd, wd, bd, sd = dev(x), dev(w), dev(bias), dev(st)
    say(f"split/resume {io}")
    u = mscan.conv1d_fwd(xd, wd, bd, sd)
    for k in (1, 3, 8, 100, 202):
        state = sd.clone()
        u1 = mscan.conv1d_fwd(xd[..., :k].contiguous(), wd, bd, state, state_out=state, return_state=True)[0]
        u2 = mscan.conv1d_fwd(xd[..., k:].contiguous(), wd, bd, state)
        assert torch.equal(torch.cat([u1, u2], dim=-1), u), k


def test_conv_full_size_sampled():
    """The 1.4B-layer shape (b4 d4096 L8192, bf16): three whole rows checked against the oracle."""
    x, w, bias, _ = conv_inputs(4, 4096, 8192, 4, "bf16", seed=0)
    say("full size")
    u = mscan.conv1d_fwd(dev(x), dev(w), dev(bias))
    rows = [(0, 0), (1, 2049), (3, 4095)]
    for bb, dd in rows:
        ur = oracle.conv1d_fwd(x[bb:bb + 1, dd:dd + 1], w[dd:dd + 1], bias[dd:dd + 1])
        rep = err_report(u[bb:bb + 1, dd:dd + 1].float().cpu(), ur)
        assert rep["max_rel"] <= TOL["bf16"], (bb, dd, rep)
