"""GPU parity at the largest sizes the C ABI accepts, where the kernels' 32-bit offsets and grid
sizes reach their limits, against the fp64 oracle on sampled rows / heads:

* forward: 64 * (L + 8) * 2 bytes < 2^31 for bf16 rows, i.e. L = 2^24 - 9 = 16777207 tokens (one
  64-channel group, so the plan cuts it into 256 time chunks: the carry and fix-up run at the limit
  too; L is not a multiple of 64, so the last tile is ragged);
* SSD: nheads * headdim = 2^24 (65536 heads of 256), where a chunk's 64 token rows of x and y
  span 63 * 2^25 + 512 bytes, just under 2^31; 100 tokens (a full and a ragged chunk);
* decode step: batch 262140 (65535 grid rows of four batch rows).

Tolerance: the bf16 bar, 1e-2 (max error over max(|ref|, rms)), on y and the final state.  Each
test needs a few GB of device memory and of host memory for its inputs."""
import sys

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_55_amd as mscan
from workloads import err_report, forward_inputs, max_rel_err, ssd_inputs, step_initial, step_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-2


def say(msg):
    print(f"[maxsize] {msg}", flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.to(DEV)


def check(name, got, ref):
    rep = err_report(got, ref)
    say(f"  {name}: {rep}")
    assert rep["max_rel"] <= TOL, (name, rep)


def test_forward_longest_row():
    L = (1 << 24) - 9
    assert 64 * (L + 8) * 2 < (1 << 31) <= 64 * (L + 9) * 2
    say(f"forward at L = {L}: generating inputs")
    inp = forward_inputs(batch=1, dim=64, dstate=16, seqlen=L, io="bf16", gated=False, seed=11)
    a = {k: dev(v) for k, v in inp.items()}
    say("forward: GPU run (default plan)")
    y, fs = mscan.scan_fwd(a["u"], a["delta"], a["A_log"], a["B"], a["C"], D=a["D"], delta_bias=a["delta_bias"],
                           return_final_state=True)
    torch.cuda.synchronize()
    rows = [0, 37, 63]
    yg = y[0, rows].cpu()
    fg = fs[0, rows].cpu()
    del y, fs, a
    torch.cuda.empty_cache()
    say(f"forward: oracle on channels {rows}")
    sub = dict(u=inp["u"][:, rows], delta=inp["delta"][:, rows], A_log=inp["A_log"][rows], B=inp["B"], C=inp["C"],
               D=inp["D"][rows], delta_bias=inp["delta_bias"][rows])
    yr, fsr = oracle.scan_fwd(sub["u"], sub["delta"], sub["A_log"], sub["B"], sub["C"], D=sub["D"],
                              delta_bias=sub["delta_bias"])
    check("y (sampled channels, whole row)", yg, yr[0])
    check("final_state (sampled channels)", fg, fsr[0])


def test_ssd_widest_token_row():
    b, L, H, P, N = 1, 100, 1 << 16, 256, 64
    assert H * P == 1 << 24
    say(f"SSD with {H} heads of {P}: generating inputs")
    inp = ssd_inputs(b, L, H, P, N, seed=12, gated=False, initial_state=False)
    say("SSD: GPU run")
    y, fs = mscan.ssd_fwd(dev(inp["x"]), dev(inp["dt"]), dev(inp["A_log"]), dev(inp["B"]), dev(inp["C"]),
                          D=dev(inp["D"]), dt_bias=dev(inp["dt_bias"]), return_final_state=True)
    torch.cuda.synchronize()
    heads = [0, 12345, H - 1]
    yg = y[:, :, heads].cpu()
    fg = fs[:, heads].cpu()
    del y, fs
    torch.cuda.empty_cache()
    say(f"SSD: oracle on heads {heads}")
    yr, fsr = oracle.ssd_fwd(inp["x"][:, :, heads], inp["dt"][:, :, heads], inp["A_log"][heads], inp["B"],
                             inp["C"], D=inp["D"][heads], dt_bias=inp["dt_bias"][heads])
    check("y (sampled heads)", yg, yr)
    check("final_state (sampled heads)", fg, fsr)


def test_step_largest_batch():
    b, d, n = 262140, 64, 16
    say(f"decode step at batch {b}")
    init = step_initial(None, batch=b, dim=d, dstate=n)
    s = step_inputs(None, 0, batch=b, dim=d, dstate=n, io="bf16", gated=True)
    st = init["state"].to(DEV)
    y = mscan.scan_step(st, dev(s["x"]), dev(s["dt"]), dev(init["A_log"]), dev(s["B"]), dev(s["C"]),
                        D=dev(init["D"]), z=dev(s["z"]), dt_bias=dev(init["dt_bias"]))
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 65535, 131071, b - 4, b - 1])
    yr, stn = oracle.scan_step(init["state"][rows], s["x"][rows], s["dt"][rows], init["A_log"], s["B"][rows],
                               s["C"][rows], D=init["D"], z=s["z"][rows], dt_bias=init["dt_bias"])
    check("y (sampled batch rows)", y[rows.to(DEV)].cpu(), yr)
    check("state (sampled batch rows)", st[rows.to(DEV)].cpu(), stn)
    assert max_rel_err(st[-1].cpu(), stn[-1]) <= TOL
