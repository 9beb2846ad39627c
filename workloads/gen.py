"""Seeded input generation for the selective-scan workloads.

Every tensor is drawn from its own numpy PCG64 stream keyed by
``SeedSequence(seed, spawn_key=(tensor_key, block))``; large tensors are cut
into blocks of whole rows (about 2^20 elements each) with one stream per block,
so generation runs in parallel threads and stays reproducible regardless of the
thread count.  Draws are float32; bfloat16 inputs are the round-to-nearest-even
rounding of those draws (torch CPU conversion).  All outputs are CPU tensors.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Union

import numpy as np
import torch

from .configs import Config, get_config

# stream keys, fixed order
(K_U, K_DELTA, K_Z, K_B, K_C, K_D, K_BIAS, K_STATE, K_STEPS, K_DY, K_DFS, K_CONVW, K_CONVB, K_CONVS,
 K_SSDA, K_ALOG) = range(16)
_BLOCK_ELEMS = 1 << 20


def _threads(threads: Optional[int]) -> int:
    if threads:
        return int(threads)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, key: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _normal_rows(seed: int, key: tuple, rows: int, L: int, io: str, std: float = 1.0,
                 threads: Optional[int] = None) -> torch.Tensor:
    """(rows, L) tensor of N(0, std^2) draws in the io dtype."""
    dtype = torch.float32 if io == "f32" else torch.bfloat16
    out = torch.empty((rows, L), dtype=dtype)
    if rows == 0 or L == 0:
        return out
    block_rows = max(1, _BLOCK_ELEMS // L)
    nblk = math.ceil(rows / block_rows)

    def work(i: int) -> None:
        r0 = i * block_rows
        r1 = min(rows, r0 + block_rows)
        tmp = _gen(seed, key + (i,)).standard_normal((r1 - r0, L), dtype=np.float32)
        if std != 1.0:
            tmp *= np.float32(std)
        out[r0:r1] = torch.from_numpy(tmp).to(dtype)

    nt = _threads(threads)
    if nblk == 1 or nt == 1:
        for i in range(nblk):
            work(i)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(nblk)))
    return out


def a_log_s4d_real(dim: int, dstate: int) -> torch.Tensor:
    """float32(log(1..N)) for every channel, shape (dim, dstate)."""
    row = np.log(np.arange(1, dstate + 1, dtype=np.float64)).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(np.broadcast_to(row, (dim, dstate))).copy())


def a_log_learned(seed: int, dim: int, dstate: int, lo: float = -6.0, hi: float = 3.0) -> torch.Tensor:
    """float32 A_log ~ U[lo, hi] per (channel, state): a learned-range A_log (|A| = e^-6 .. e^3),
    where the S4D-Real log(1..N) is only the initialisation."""
    return torch.from_numpy(_gen(seed, (K_ALOG, 0)).uniform(lo, hi, size=(dim, dstate)).astype(np.float32))


def make_a_log(a_log: str, seed: int, dim: int, dstate: int) -> torch.Tensor:
    if a_log == "s4d":
        return a_log_s4d_real(dim, dstate)
    if a_log == "learned":
        return a_log_learned(seed, dim, dstate)
    raise ValueError(f"a_log must be 's4d' or 'learned', not {a_log!r}")


def delta_bias_init(seed: int, dim: int, lo: float = 0.001, hi: float = 0.1) -> torch.Tensor:
    """float32(log(expm1(U[lo, hi]))) per channel: softplus of it is uniform on [lo, hi]."""
    uni = _gen(seed, (K_BIAS, 0)).uniform(lo, hi, size=dim)
    return torch.from_numpy(np.log(np.expm1(uni)).astype(np.float32))


def forward_inputs(cfg: Union[int, Config, None] = None, *, seed: int = 0, batch: int = None, dim: int = None,
                   dstate: int = None, seqlen: int = None, io: str = None, gated: bool = None,
                   has_D: bool = None, has_bias: bool = None, initial_state: bool = False,
                   a_log: str = "s4d", bias_range=(0.001, 0.1), delta_std: float = 1.0,
                   threads: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of one forward scan as CPU tensors.

    Either a config (index or Config) or explicit shape keywords (which override
    the config's values).  Keys: u, delta, z, B, C (io dtype), A_log, D,
    delta_bias (float32), initial_state (float32 or None).

    Value regime (defaults: the workloads' distributions):
      a_log       "s4d" (log(1..N) per channel) or "learned" (U[-6, 3] per (channel, state));
      bias_range  softplus(delta_bias) ~ U[lo, hi] per channel; (1e-4, 2e-4) gives the
                  Delta ~ 1/L initialisation of the Mamba notes (训练策略) at L ~ 8192;
      delta_std   delta ~ N(0, delta_std^2); 0 makes delta exactly zero (Delta = softplus(bias)).
    """
    c = get_config(cfg) if isinstance(cfg, int) else cfg
    pick = lambda v, attr, dflt: v if v is not None else (getattr(c, attr) if c is not None else dflt)
    b = pick(batch, "batch", 1)
    d = pick(dim, "dim", 64)
    n = pick(dstate, "dstate", 16)
    L = pick(seqlen, "seqlen", 256)
    io_ = pick(io, "io", "bf16")
    gated_ = pick(gated, "gated", True)
    hasD = pick(has_D, "has_D", True)
    hasB = pick(has_bias, "has_bias", True)
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["u"] = _normal_rows(seed, (K_U,), b * d, L, io_, threads=threads).view(b, d, L)
    if delta_std == 0.0:
        out["delta"] = torch.zeros((b, d, L), dtype=torch.float32 if io_ == "f32" else torch.bfloat16)
    else:
        out["delta"] = _normal_rows(seed, (K_DELTA,), b * d, L, io_, std=delta_std, threads=threads).view(b, d, L)
    out["z"] = _normal_rows(seed, (K_Z,), b * d, L, io_, threads=threads).view(b, d, L) if gated_ else None
    out["B"] = _normal_rows(seed, (K_B,), b * n, L, io_, threads=threads).view(b, n, L)
    out["C"] = _normal_rows(seed, (K_C,), b * n, L, io_, threads=threads).view(b, n, L)
    out["A_log"] = make_a_log(a_log, seed, d, n)
    out["D"] = torch.from_numpy(_gen(seed, (K_D, 0)).standard_normal(d, dtype=np.float32)) if hasD else None
    out["delta_bias"] = delta_bias_init(seed, d, *bias_range) if hasB else None
    out["initial_state"] = (_normal_rows(seed, (K_STATE,), b * d, n, "f32", std=0.1, threads=threads)
                            .view(b, d, n) if initial_state else None)
    return out


def step_initial(cfg: Union[int, Config, None] = None, *, seed: int = 0, batch: int = None, dim: int = None,
                 dstate: int = None, a_log: str = "s4d", bias_range=(0.001, 0.1),
                 threads: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Decode-step state and parameters: state (b,d,n) fp32 ~ N(0, 0.1^2), A_log, D, dt_bias
    (a_log and bias_range as in forward_inputs)."""
    c = get_config(cfg) if isinstance(cfg, int) else cfg
    b = batch if batch is not None else c.batch
    d = dim if dim is not None else c.dim
    n = dstate if dstate is not None else c.dstate
    return {
        "state": _normal_rows(seed, (K_STATE,), b * d, n, "f32", std=0.1, threads=threads).view(b, d, n),
        "A_log": make_a_log(a_log, seed, d, n),
        "D": torch.from_numpy(_gen(seed, (K_D, 0)).standard_normal(d, dtype=np.float32)),
        "dt_bias": delta_bias_init(seed, d, *bias_range),
    }


def step_inputs(cfg: Union[int, Config, None], k: int, *, seed: int = 0, batch: int = None, dim: int = None,
                dstate: int = None, io: str = None, gated: bool = None, dt_std: float = 1.0,
                threads: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Fresh per-step inputs of decode step k: x, dt, z (b,d) and B, C (b,n) in the io dtype;
    dt ~ N(0, dt_std^2) (0: exactly zero)."""
    c = get_config(cfg) if isinstance(cfg, int) else cfg
    b = batch if batch is not None else c.batch
    d = dim if dim is not None else c.dim
    n = dstate if dstate is not None else c.dstate
    io_ = io if io is not None else c.io
    g_ = gated if gated is not None else c.gated
    key = (K_STEPS, int(k))
    return {
        "x": _normal_rows(seed, key + (0,), b, d, io_, threads=threads),
        "dt": (_normal_rows(seed, key + (1,), b, d, io_, std=dt_std, threads=threads) if dt_std != 0.0
               else torch.zeros((b, d), dtype=torch.float32 if io_ == "f32" else torch.bfloat16)),
        "z": _normal_rows(seed, key + (2,), b, d, io_, threads=threads) if g_ else None,
        "B": _normal_rows(seed, key + (3,), b, n, io_, threads=threads),
        "C": _normal_rows(seed, key + (4,), b, n, io_, threads=threads),
    }


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU tensor (bf16/fp16/fp32/fp64) to float64 numpy."""
    t = t.detach().to("cpu")
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.to(torch.float32)
    return t.numpy().astype(np.float64)


def backward_inputs(batch: int, dim: int, dstate: int, seqlen: int, io: str, *, seed: int = 0,
                    d_final_state: bool = False, threads: Optional[int] = None):
    """Output gradients for a backward pass: dy (batch, dim, L) ~ N(0, 1) in the io dtype and,
    if asked, dL/d(final state) (batch, dim, dstate) ~ N(0, 1) float32.  Returns (dy, dfs or None)."""
    dy = _normal_rows(seed, (K_DY,), batch * dim, seqlen, io, threads=threads).view(batch, dim, seqlen)
    dfs = None
    if d_final_state:
        dfs = _normal_rows(seed, (K_DFS,), batch * dim, dstate, "f32", threads=threads).view(batch, dim, dstate)
    return dy, dfs


def conv_inputs(batch: int, dim: int, seqlen: int, K: int, io: str, *, seed: int = 0, state: bool = False,
                threads: Optional[int] = None):
    """Inputs of the causal conv1d: x (batch, dim, L) ~ N(0, 1) in the io dtype, weight (dim, K) ~
    N(0, 1/K) float32, bias (dim,) ~ N(0, 0.1^2) float32, and optionally a conv state
    (batch, dim, K-1) ~ N(0, 1) in the io dtype.  Returns (x, weight, bias, state or None)."""
    x = _normal_rows(seed, (K_U,), batch * dim, seqlen, io, threads=threads).view(batch, dim, seqlen)
    w = torch.from_numpy(_gen(seed, (K_CONVW, 0)).standard_normal((dim, K), dtype=np.float32)
                         * np.float32(1.0 / math.sqrt(K)))
    bias = torch.from_numpy(_gen(seed, (K_CONVB, 0)).standard_normal(dim, dtype=np.float32) * np.float32(0.1))
    st = None
    if state:
        st = _normal_rows(seed, (K_CONVS,), batch * dim, K - 1, io, threads=threads).view(batch, dim, K - 1)
    return x, w, bias, st


def ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, *, seed: int = 0,
               gated: bool = False, initial_state: bool = False, threads: Optional[int] = None,
               x_std: float = 1.0, dt_std: float = 1.0, bc_std: Optional[float] = None,
               bias_range: tuple = (1e-3, 1e-1)):
    """Inputs of the multi-head SSM (state-space-duality form), token-major, bf16 io:
    x, z (batch, L, H, P) ~ N(0, 1) (x ~ N(0, x_std^2)); dt (batch, L, H) ~ N(0, dt_std^2); B, C
    (batch, L, N) ~ N(0, 1/N) (a readout over N states then has unit scale; N(0, bc_std^2) when
    given); A_log = log(U[1, 16]) per head; D ~ N(0, 1); dt_bias = log(expm1(U[bias_range])) per
    head (softplus(dt_bias) uniform on bias_range, default [1e-3, 1e-1]); initial_state
    (batch, H, P, N) ~ N(0, 0.1^2)."""
    bcs = 1.0 / math.sqrt(dstate) if bc_std is None else bc_std
    x = _normal_rows(seed, (K_U,), batch * seqlen, nheads * headdim, "bf16", std=x_std, threads=threads)
    dt = _normal_rows(seed, (K_DELTA,), batch * seqlen, nheads, "bf16", std=dt_std, threads=threads)
    B = _normal_rows(seed, (K_B,), batch * seqlen, dstate, "bf16", std=bcs, threads=threads)
    C = _normal_rows(seed, (K_C,), batch * seqlen, dstate, "bf16", std=bcs, threads=threads)
    z = (_normal_rows(seed, (K_Z,), batch * seqlen, nheads * headdim, "bf16", threads=threads)
         .view(batch, seqlen, nheads, headdim) if gated else None)
    A_log = torch.from_numpy(np.log(_gen(seed, (K_SSDA, 0)).uniform(1.0, 16.0, size=nheads)).astype(np.float32))
    D = torch.from_numpy(_gen(seed, (K_D, 0)).standard_normal(nheads, dtype=np.float32))
    u = _gen(seed, (K_BIAS, 0)).uniform(bias_range[0], bias_range[1], size=nheads)
    dt_bias = torch.from_numpy(np.log(np.expm1(u)).astype(np.float32))
    h0 = None
    if initial_state:
        h0 = torch.from_numpy(_gen(seed, (K_STATE, 0)).standard_normal((batch, nheads, headdim, dstate),
                                                                        dtype=np.float32) * np.float32(0.1))
    return dict(x=x.view(batch, seqlen, nheads, headdim), dt=dt.view(batch, seqlen, nheads), A_log=A_log,
                B=B.view(batch, seqlen, dstate), C=C.view(batch, seqlen, dstate), D=D, z=z, dt_bias=dt_bias,
                initial_state=h0)
