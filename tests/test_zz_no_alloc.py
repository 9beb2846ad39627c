"""The allocation-free forward (mamba_scan_fwd_noalloc, static per-GPU scratch) against the
workspace forward (mamba_scan_fwd) through the C ABI: same plan, same kernels, so the results
must be identical bit for bit, and within the io tolerance of the fp64 oracle.  Two calls in a
row, the second smaller (it reuses the scratch the first left behind), a d_state-32 call whose
readout sum over the two state passes lives in the scratch, a head/tail-plan call whose tail
keeps its y in fp32 in the scratch, and a call on a side stream."""
import sys

import pytest
import torch

import oracle
import selective_state_space_55_amd as mscan
from workloads import forward_inputs, max_rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 1e-2}


def say(msg):
    print(f"[noalloc] {msg}", flush=True)
    sys.stdout.flush()


def run_both(inp, stream=None):
    a = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    b, d, L = a["u"].shape
    n = a["A_log"].shape[1]
    y_ref, fs_ref = mscan.scan_fwd(a["u"], a["delta"], a["A_log"], a["B"], a["C"], D=a["D"], z=a["z"],
                                   delta_bias=a["delta_bias"], initial_state=a["initial_state"],
                                   return_final_state=True)
    # outputs of the no-alloc call are pre-filled with garbage: every element must be written
    y = torch.full((b, d, L), float("nan"), dtype=a["u"].dtype, device=DEV)
    fs = torch.full((b, d, n), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    mscan.scan_fwd_noalloc(a["u"], a["delta"], a["A_log"], a["B"], a["C"], out=y, D=a["D"], z=a["z"],
                           delta_bias=a["delta_bias"], initial_state=a["initial_state"], final_state=fs,
                           stream=stream)
    torch.cuda.synchronize()
    return y.cpu(), fs.cpu(), y_ref.cpu(), fs_ref.cpu()


def check(inp, io, stream=None):
    y, fs, y_ref, fs_ref = run_both(inp, stream)
    assert torch.equal(y.view(torch.int16) if io == "bf16" else y.view(torch.int32),
                       y_ref.view(torch.int16) if io == "bf16" else y_ref.view(torch.int32))
    assert torch.equal(fs.view(torch.int32), fs_ref.view(torch.int32))
    yr, fsr = oracle.scan_fwd(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                              delta_bias=inp["delta_bias"], initial_state=inp["initial_state"])
    ey, ef = max_rel_err(y, yr), max_rel_err(fs, fsr)
    say(f"  y {ey:.3e}  final_state {ef:.3e}")
    assert ey <= TOL[io] and ef <= TOL[io]


def test_two_calls_second_smaller():
    # b1 d128 L4096: two channel groups, so the plan scans 8 time chunks (chunk carry in the scratch)
    big = forward_inputs(batch=1, dim=128, dstate=16, seqlen=4096, io="bf16", initial_state=True, seed=1)
    assert mscan.fwd_workspace_size(1, 128, 16, 4096, mscan.BF16) > 0
    say("call 1: b1 d128 L4096 bf16 (chunked)")
    check(big, "bf16")
    small = forward_inputs(batch=1, dim=64, dstate=16, seqlen=2048, io="bf16", initial_state=True, seed=2)
    assert mscan.fwd_workspace_size(1, 64, 16, 2048, mscan.BF16) > 0
    say("call 2: b1 d64 L2048 bf16 (chunked, smaller, scratch left by call 1)")
    check(small, "bf16")


def test_head_tail_fp32_tail_y_in_scratch():
    # b3 d3072 L1600: 144 channel groups, so the plan splits each row into a head and a tail whose
    # y is kept in fp32 (in the scratch) until the fix-up rounds it once
    inp = forward_inputs(batch=3, dim=3072, dstate=16, seqlen=1600, io="bf16", initial_state=True, seed=7)
    say("call 1: b3 d3072 L1600 bf16 (head/tail, fp32 tail y in the scratch)")
    check(inp, "bf16")
    small = forward_inputs(batch=1, dim=128, dstate=16, seqlen=4096, io="bf16", initial_state=True, seed=8)
    say("call 2: b1 d128 L4096 bf16 (chunked, smaller)")
    check(small, "bf16")


def test_wide_state_readout_sum_in_scratch():
    inp = forward_inputs(batch=2, dim=64, dstate=32, seqlen=1000, io="f32", initial_state=True, seed=3)
    say("d_state 32 f32 (readout sum over two passes in the scratch)")
    check(inp, "f32")
    small = forward_inputs(batch=1, dim=64, dstate=20, seqlen=300, io="f32", seed=4)
    say("d_state 20 f32, smaller")
    check(small, "f32")


def test_side_stream_and_no_workspace_needed():
    s = torch.cuda.Stream()
    inp = forward_inputs(batch=1, dim=128, dstate=16, seqlen=2048, io="f32", seed=5)
    say("side stream, chunked")
    check(inp, "f32", stream=s)
    one_pass = forward_inputs(batch=4, dim=2048, dstate=16, seqlen=256, io="bf16", seed=6)
    assert mscan.fwd_workspace_size(4, 2048, 16, 256, mscan.BF16) == 0
    say("one pass, no scratch used")
    check(one_pass, "bf16")
