"""Seeded input generators and the comparison metric (CPU only)."""
import math

import numpy as np
import pytest
import torch

import workloads
from workloads import CONFIGS, forward_inputs, max_rel_err, step_initial, step_inputs


def test_configs_match_the_five_workloads():
    c = CONFIGS
    assert (c[0].batch, c[0].dim, c[0].dstate, c[0].seqlen, c[0].io) == (1, 64, 16, 256, "f32")
    assert (c[1].batch, c[1].dim, c[1].dstate, c[1].seqlen, c[1].io) == (8, 1536, 16, 2048, "bf16")
    assert (c[2].batch, c[2].dim, c[2].dstate, c[2].seqlen, c[2].io) == (4, 4096, 16, 8192, "bf16")
    assert (c[3].batch, c[3].dim, c[3].dstate, c[3].seqlen, c[3].gated) == (1, 2048, 16, 1 << 20, False)
    assert (c[4].batch, c[4].dim, c[4].dstate, c[4].steps) == (256, 5120, 16, 1024)
    assert c[0].tol == 1e-4 and all(c[k].tol == 1e-2 for k in (1, 2, 3, 4))
    # algorithmic bytes: 8 B per token-channel at bf16 gated (+ B, C, params, final state)
    assert abs(c[2].algorithmic_bytes() / 1e6 - 1077.2) < 0.5
    assert abs(c[3].algorithmic_bytes() / 1e9 - 12.95) < 0.01


def test_forward_inputs_deterministic_and_thread_independent():
    a = forward_inputs(0, threads=1)
    b = forward_inputs(0, threads=4)
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            assert torch.equal(a[k], b[k]), k
    assert a["u"].shape == (1, 64, 256) and a["u"].dtype == torch.float32
    assert a["B"].shape == (1, 16, 256)
    assert a["A_log"].shape == (64, 16)
    assert torch.allclose(a["A_log"][5], torch.log(torch.arange(1, 17, dtype=torch.float64)).float())


def test_bias_softplus_range_and_bf16_rounding():
    x = forward_inputs(batch=2, dim=300, dstate=16, seqlen=40, io="bf16")
    sp = np.logaddexp(0.0, x["delta_bias"].double().numpy())
    assert sp.min() >= 0.001 * (1 - 1e-6) and sp.max() <= 0.1 * (1 + 1e-6)
    assert x["u"].dtype == torch.bfloat16
    # bf16 values are the RNE rounding of the float32 draws of the same stream
    f = forward_inputs(batch=2, dim=300, dstate=16, seqlen=40, io="f32")
    assert torch.equal(f["u"].to(torch.bfloat16), x["u"])
    assert 0.9 < float(f["u"].std()) < 1.1


def test_step_inputs_fresh_per_step():
    s0 = step_inputs(4, 0, batch=2, dim=8, dstate=16)
    s1 = step_inputs(4, 1, batch=2, dim=8, dstate=16)
    assert not torch.equal(s0["x"], s1["x"])
    assert torch.equal(s0["x"], step_inputs(4, 0, batch=2, dim=8, dstate=16)["x"])
    st = step_initial(4, batch=64, dim=64, dstate=16)
    assert st["state"].shape == (64, 64, 16)
    assert 0.09 < float(st["state"].std()) < 0.11


def test_max_rel_err_metric():
    r = np.array([1.0, -2.0, 0.0, 4.0])
    assert max_rel_err(r, r) == 0.0
    g = r.copy()
    g[2] = 0.01
    rms = math.sqrt(np.mean(r * r))
    assert abs(max_rel_err(g, r) - 0.01 / rms) < 1e-15
    g = r.copy()
    g[0] = np.nan
    assert max_rel_err(g, r) == math.inf
    rn = r.copy()
    rn[0] = np.nan
    assert max_rel_err(rn, rn) == 0.0
    assert max_rel_err(np.zeros(3), np.zeros(3)) == 0.0
