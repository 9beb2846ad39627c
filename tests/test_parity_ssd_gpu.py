"""GPU parity of the multi-head SSM with a scalar decay per head (state-space-
duality form, mamba_ssd_fwd, matrix cores) against the fp64 oracle: ragged
lengths (partial last chunk), one-token and empty sequences, d_state 64 and
128, head dims 32 to 256 (32- and 64-channel slices), gate / no gate, initial state, both input terms, softplus off; repeat
runs are identical; a split at a chunk boundary resumes bit for bit and at any
other token within tolerance; the full-size layer on sampled heads.

Tolerance: the products take bf16 operands with fp32 accumulation: x, B, C as
given, the masked decay matrix rounded to bf16, and the two operands that carry
fp32 values -- the state that C reads and x times its decayed weight in the
state update -- each split as bf16 hi + bf16 of the rest (~2^-17 relative).  So
the bar is the bf16 one used throughout, 1e-2 (max error over max(|ref|, rms)).
The small-Delta cases run where the weight alone is ~1e-4 and a state keeps its
inputs over many chunks."""
import sys

import pytest
import torch

import oracle
import selective_state_space_55_amd as mscan
from workloads import err_report, max_rel_err, ssd_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-2


def say(msg):
    print(f"[ssd] {msg}", flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.to(DEV)


def gpu(inp, softplus=True, disc="zoh", h0=None):
    y, fs = mscan.ssd_fwd(dev(inp["x"]), dev(inp["dt"]), dev(inp["A_log"]), dev(inp["B"]), dev(inp["C"]),
                          D=dev(inp["D"]), z=dev(inp["z"]), dt_bias=dev(inp["dt_bias"]),
                          initial_state=dev(inp["initial_state"] if h0 is None else h0), dt_softplus=softplus,
                          return_final_state=True, discretization=disc)
    torch.cuda.synchronize()
    return y.cpu(), fs.cpu()


def ref(inp, softplus=True, disc="zoh"):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A_log"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                          dt_bias=inp["dt_bias"], initial_state=inp["initial_state"], dt_softplus=softplus,
                          discretization=disc)


def check(name, got, want):
    rep = err_report(got, want)
    say(f"  {name}: {rep}")
    assert rep["max_rel"] <= TOL, (name, rep)


CASES = [  # (batch, L, H, N, gated, h0, disc, softplus)
    (1, 64, 1, 64, False, False, "zoh", True),
    (2, 200, 3, 128, True, True, "zoh", True),
    (1, 1, 2, 64, True, True, "zoh", True),
    (1, 129, 2, 128, False, True, "euler", True),
    (2, 1000, 4, 128, True, False, "zoh", True),
    (1, 333, 3, 64, True, True, "euler", True),
    (1, 150, 2, 128, False, True, "zoh", False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}L{c[1]}H{c[2]}N{c[3]}{c[6]}" + ("g" if c[4] else "")
                                            + ("" if c[7] else "-nosp") for c in CASES])
def test_ssd_vs_oracle(case):
    b, L, H, N, gated, h0, disc, sp = case
    inp = ssd_inputs(b, L, H, 64, N, seed=L + H + N, gated=gated, initial_state=h0)
    if not sp:
        inp["dt"] = (inp["dt"].float().abs() * 0.05).to(torch.bfloat16)
        inp["dt_bias"] = inp["dt_bias"].abs() * 0.01
    say(f"case {case}")
    y, fs = gpu(inp, sp, disc)
    yr, fsr = ref(inp, sp, disc)
    check("y", y, yr)
    check("final_state", fs, fsr)


@pytest.mark.parametrize("P,N,disc", [(128, 128, "zoh"), (128, 64, "euler"), (192, 64, "zoh"), (256, 128, "zoh"),
                                     (32, 128, "zoh"), (96, 64, "euler"), (160, 128, "zoh")])
def test_ssd_head_dims_vs_oracle(P, N, disc):
    """Head dims other than 64: each head runs as slices of 32 or 64 channels sharing its decay."""
    b, L, H = 2, 150, 2
    inp = ssd_inputs(b, L, H, P, N, seed=P + N, gated=True, initial_state=True)
    say(f"head dim {P}, N {N}, {disc}")
    y, fs = gpu(inp, True, disc)
    yr, fsr = ref(inp, True, disc)
    check("y", y, yr)
    check("final_state", fs, fsr)


@pytest.mark.parametrize("N,disc,gated", [(128, "zoh", True), (64, "euler", False)])
def test_ssd_many_heads_vs_oracle(N, disc, gated):
    """More (batch, head) pairs than the GPU has CUs (260 workgroups), with a ragged last chunk."""
    b, L, H = 2, 70, 130
    inp = ssd_inputs(b, L, H, 64, N, seed=H + N, gated=gated, initial_state=True)
    say(f"{b * H} heads, N {N}, {disc}")
    y, fs = gpu(inp, True, disc)
    yr, fsr = ref(inp, True, disc)
    check("y", y, yr)
    check("final_state", fs, fsr)


def test_ssd_head_of_128_equals_two_heads_of_64():
    """A head of dim 128 is two heads of dim 64 with the same dt, A, D: identical results bit for bit
    (same memory layout; dt, A_log, D, dt_bias repeated per half)."""
    b, L, H, P, N = 1, 200, 3, 128, 128
    inp = ssd_inputs(b, L, H, P, N, seed=3, gated=True, initial_state=True)
    y1, fs1 = gpu(inp)
    two = dict(x=inp["x"].view(b, L, 2 * H, 64), z=inp["z"].view(b, L, 2 * H, 64),
               dt=inp["dt"].repeat_interleave(2, dim=2).contiguous(), B=inp["B"], C=inp["C"],
               A_log=inp["A_log"].repeat_interleave(2), D=inp["D"].repeat_interleave(2),
               dt_bias=inp["dt_bias"].repeat_interleave(2),
               initial_state=inp["initial_state"].view(b, 2 * H, 64, N))
    y2, fs2 = gpu(two)
    assert torch.equal(y1.view(torch.int16), y2.view(b, L, H, P).view(torch.int16))
    assert torch.equal(fs1, fs2.view(b, H, P, N))


def test_ssd_empty_sequence():
    inp = ssd_inputs(2, 0, 3, 64, 64, seed=1, initial_state=True)
    say("empty")
    y, fs = gpu(inp)
    assert y.shape == (2, 0, 3, 64)
    assert torch.equal(fs, inp["initial_state"])


def test_ssd_deterministic():
    inp = ssd_inputs(2, 300, 4, 64, 128, seed=2, gated=True, initial_state=True)
    say("determinism")
    y1, f1 = gpu(inp)
    y2, f2 = gpu(inp)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("k", [128, 100])
def test_ssd_split_resume(k):
    """Split at token k: at a chunk boundary (k = 128) the resumed run is bit-identical (the state
    crosses the call in fp32 exactly as it crosses a chunk); elsewhere it is within tolerance."""
    L = 300
    inp = ssd_inputs(1, L, 3, 64, 128, seed=3, gated=True, initial_state=True)
    say(f"split at {k}")
    y, fs = gpu(inp)
    first = {kk: (v[:, :k].contiguous() if kk in ("x", "dt", "B", "C", "z") and v is not None else v)
             for kk, v in inp.items()}
    second = {kk: (v[:, k:].contiguous() if kk in ("x", "dt", "B", "C", "z") and v is not None else v)
              for kk, v in inp.items()}
    y1, f1 = gpu(first)
    y2, f2 = gpu(second, h0=f1)
    yy = torch.cat([y1, y2], dim=1)
    if k % 64 == 0:
        assert torch.equal(yy, y) and torch.equal(f2, fs)
    else:
        assert max_rel_err(yy, y.double()) <= TOL and max_rel_err(f2, fs.double()) <= TOL


def test_ssd_full_size_sampled_heads():
    """The benchmark layer (batch 4, L 8192, 64 heads of 64, d_state 128): three (batch, head) pairs
    checked against the oracle over the whole sequence."""
    b, L, H, N = 4, 8192, 64, 128
    inp = ssd_inputs(b, L, H, 64, N, seed=0)
    say("full size")
    y, fs = gpu(inp)
    for bb, hh in [(0, 0), (1, 33), (3, 63)]:
        sub = dict(x=inp["x"][bb:bb + 1, :, hh:hh + 1], dt=inp["dt"][bb:bb + 1, :, hh:hh + 1],
                   A_log=inp["A_log"][hh:hh + 1], B=inp["B"][bb:bb + 1], C=inp["C"][bb:bb + 1],
                   D=inp["D"][hh:hh + 1], z=None, dt_bias=inp["dt_bias"][hh:hh + 1], initial_state=None)
        yr, fr = ref(sub)
        check(f"y b{bb} h{hh}", y[bb:bb + 1, :, hh:hh + 1], yr)
        check(f"final b{bb} h{hh}", fs[bb:bb + 1, hh:hh + 1], fr)


@pytest.mark.parametrize("x_std,disc", [(1.0, "zoh"), (0.01, "zoh"), (0.01, "euler")])
def test_ssd_small_delta(x_std, disc):
    """Delta ~ 1e-4 (softplus(dt_bias) in [1e-4, 2e-4], dt ~ N(0, 0.1^2)): the state update's weight
    exp(cum_Q - cum_j) w_j is then ~2^-13, at the bottom of fp16's normal range, and with x ~ N(0, 0.01^2)
    the product x w is ~1e-6 (fp16 subnormal, 4 bits) unless the chunk is scaled; B, C ~ N(0, 1) and
    4096 tokens, so the state keeps its inputs over the whole sequence (|A| Delta L <= 6.5)."""
    b, L, H, N = 1, 4096, 4, 128
    inp = ssd_inputs(b, L, H, 64, N, seed=7, gated=True, initial_state=True, x_std=x_std, dt_std=0.1,
                     bc_std=1.0, bias_range=(1e-4, 2e-4))
    say(f"small Delta x_std={x_std} {disc}")
    y, fs = gpu(inp, True, disc)
    yr, fsr = ref(inp, True, disc)
    check("y", y, yr)
    check("final_state", fs, fsr)
