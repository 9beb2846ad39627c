"""The five workload shapes of the selective scan.

Shapes follow the Mamba layer sizes with expand factor 2 (d_inner = 2 d_model;
Mamba concept page, compassingai.com, §4.2, and the MAMBA walkthrough,
x-humanoid.csdn.net, §6 usage snippet) and d_state = 16 (Mamba notes,
awesome.papernotes.org, 设计 2).  Value distributions:

* u, delta, z, B, C ~ N(0, 1) drawn in float32, then rounded to the io dtype
  (round-to-nearest-even for bfloat16);
* A_log = float32(log(1..N)) for every channel (S4D-Real init; State space
  models and Mamba, jonathanding.github.io, §1.5);
* D ~ N(0, 1) float32 per channel;
* delta_bias = float32(log(expm1(U[0.001, 0.1]))) per channel, so that
  softplus(bias) is uniform on [0.001, 0.1] (the "small Delta at start"
  initialisation of the Mamba notes, 训练策略);
* decode state ~ N(0, 0.1^2) float32 (standard deviation 0.1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    kind: str            # "fwd" (full-sequence scan) or "step" (chained decode steps)
    batch: int
    dim: int
    dstate: int
    seqlen: int = 0      # fwd only
    steps: int = 0       # step only
    io: str = "bf16"     # "f32" or "bf16"
    gated: bool = True
    has_D: bool = True
    has_bias: bool = True
    softplus: bool = True
    final_state: bool = True
    tol: float = 1e-2    # max relative error bound (1e-4 for fp32 io, 1e-2 for bf16 io)
    notes: str = ""

    @property
    def token_channels(self) -> int:
        if self.kind == "fwd":
            return self.batch * self.dim * self.seqlen
        return self.batch * self.dim * self.steps

    def io_bytes(self) -> int:
        return 4 if self.io == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move once: inputs read once, outputs written once."""
        e = self.io_bytes()
        b, d, n = self.batch, self.dim, self.dstate
        if self.kind == "fwd":
            L = self.seqlen
            per_tc = e * (3 + (1 if self.gated else 0))   # u, delta, y (+ z)
            tot = per_tc * b * d * L
            tot += 2 * e * b * n * L                      # B, C
            tot += 4 * d * n + 4 * d * (int(self.has_D) + int(self.has_bias))
            if self.final_state:
                tot += 4 * b * d * n
            return tot
        # one decode step: state read + written, x/dt/(z)/y, B/C per batch row, params
        per_bd = 2 * 4 * n + e * (3 + (1 if self.gated else 0))
        return per_bd * b * d + 2 * e * b * n + 4 * d * n + 4 * d * (int(self.has_D) + int(self.has_bias))


CONFIGS: Dict[int, Config] = {
    0: Config(0, "tiny-fp32", "fwd", 1, 64, 16, seqlen=256, io="f32", tol=1e-4,
              notes="batch 1, d_inner 64, d_state 16, L 256, fp32 io, gated, seed 0"),
    1: Config(1, "mamba-130m-layer", "fwd", 8, 1536, 16, seqlen=2048,
              notes="d_model 768 -> d_inner 1536, bf16 io, gated, final_state"),
    2: Config(2, "mamba-1.4b-layer", "fwd", 4, 4096, 16, seqlen=8192,
              notes="d_model 2048 -> d_inner 4096, bf16 io, gated, final_state"),
    3: Config(3, "million-length", "fwd", 1, 2048, 16, seqlen=1 << 20, gated=False,
              notes="ungated, bf16 io, Delta = softplus(delta + bias), bias spans softplus^-1[1e-3, 1e-1]"),
    4: Config(4, "decode-2.8b", "step", 256, 5120, 16, steps=1024,
              notes="d_inner 5120 (Mamba-2.8B-shaped), fp32 state ~ N(0, 0.1^2), 1024 chained steps"),
}


def get_config(idx: int) -> Config:
    return CONFIGS[int(idx)]


def by_name(name: str) -> Config:
    """The workload called ``name`` (e.g. ``"mamba-1.4b-layer"``)."""
    for c in CONFIGS.values():
        if c.name == name:
            return c
    raise KeyError(name)
