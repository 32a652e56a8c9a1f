"""Seeded synthetic inputs for the mLSTM forward, its backward and the decode step.

This module holds input recipes only -- shapes, distributions, seeds and the
fp32 -> bf16 rounding of inputs -- and none of the mLSTM arithmetic.  It is the one
piece shared by the HIP-side tests/benchmark and the CPU oracle side, so both
consume bit-identical values.

Workloads (xLSTM language-model layer shapes; gate pre-activations fp32):
  tiny      B=1  NH=1 S=64    d=16   chunk=16  fp32 q/k/v
  lm_125m   B=8  NH=4 S=2048  d=384  chunk=64  bf16 q/k/v
  lm_1_3b   B=4  NH=4 S=2048  d=1024 chunk=64  bf16 q/k/v
  long_ctx  B=1  NH=8 S=32768 d=256  chunk=128 bf16 q/k/v, i~ with 1% spikes at +40
  decode    batch 256, NH=4, d=512, 128 one-token steps from a random fp32 state
  slstm_125m  sLSTM B=8 NH=4 S=2048 d_h=192, bf16 recurrent matrices

Recipe (per workload, generator ``numpy.random.default_rng(seed)``):
  draw order q, k, v, i~, f~, o~ (then the spike positions, then the decode state);
  the backward's dh ~ N(0,1) comes from a generator of its own (seed + 2000), the
  block epilogue's inputs from another (seed + 3000), the sLSTM's from another
  (seed + 4000);
  normals drawn directly in float32; k scaled by 1/sqrt(d_qk) in fp32 for the
  forward workloads (decode keys are unscaled N(0,1)); q, k, v of bf16 workloads
  rounded to bf16 with round-to-nearest-even, kept here as float32 arrays that
  hold exactly representable bf16 values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd" or "step"
    B: int
    NH: int
    S: int               # tokens per sequence (fwd) or number of steps (step)
    dqk: int
    dv: int
    chunk: int           # chunk size of the parallel forward (0 for step)
    dtype: str           # "f32" or "bf16": dtype of q, k, v and h
    i_mu: float = 0.0
    i_sd: float = 1.0
    f_mu: float = 3.0
    f_sd: float = 1.0
    spike_frac: float = 0.0
    spike_value: float = 40.0
    scale_k: bool = True
    seed: int = 0

    @property
    def heads(self) -> int:
        return self.B * self.NH

    @property
    def tokens(self) -> int:
        return self.B * self.S


WORKLOADS = {
    "tiny": Workload("tiny", "fwd", 1, 1, 64, 16, 16, 16, "f32", seed=1),
    "lm_125m": Workload("lm_125m", "fwd", 8, 4, 2048, 384, 384, 64, "bf16", seed=2),
    "lm_1_3b": Workload("lm_1_3b", "fwd", 4, 4, 2048, 1024, 1024, 64, "bf16", seed=3),
    "long_ctx": Workload("long_ctx", "fwd", 1, 8, 32768, 256, 256, 128, "bf16",
                         i_mu=0.0, i_sd=8.0, f_mu=1.0, f_sd=2.0, spike_frac=0.01, seed=4),
    "decode": Workload("decode", "step", 256, 4, 128, 512, 512, 0, "bf16", scale_k=False, seed=5),
    # a key width off the matrix cores' 64-column grid (runs zero-padded to 128)
    "lm_125m_d96": Workload("lm_125m_d96", "fwd", 8, 4, 2048, 96, 96, 64, "bf16", seed=7),
    # many narrow heads: one 64-column value tile per head, where the block epilogue
    # runs inside the scan (embedding 1024 over 16 heads)
    "heads64": Workload("heads64", "fwd", 8, 16, 2048, 64, 64, 64, "bf16", seed=8),
    # sLSTM: d_qk = d_v = d_h, the cells per head (embedding 768 over 4 heads)
    "slstm_125m": Workload("slstm_125m", "slstm", 8, 4, 2048, 192, 192, 0, "bf16", seed=6),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _normal(rng, shape, mu=0.0, sd=1.0):
    z = rng.standard_normal(shape, dtype=np.float32)
    if sd != 1.0:
        z *= np.float32(sd)
    if mu != 0.0:
        z += np.float32(mu)
    return z


def fwd_inputs(w: Workload, seed: int | None = None, B: int | None = None, NH: int | None = None,
               S: int | None = None, dqk: int | None = None, dv: int | None = None):
    """Inputs of one parallel forward: dict of float32 arrays.

    q,k [B,NH,S,dqk]; v,o_pre [B,NH,S,dv]; i_pre,f_pre [B,NH,S].  Any shape field can
    be overridden (same distributions), which the parity tests use for reduced sizes.
    """
    B = w.B if B is None else B
    NH = w.NH if NH is None else NH
    S = w.S if S is None else S
    dqk = w.dqk if dqk is None else dqk
    dv = w.dv if dv is None else dv
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _normal(rng, (B, NH, S, dqk))
    k = _normal(rng, (B, NH, S, dqk))
    v = _normal(rng, (B, NH, S, dv))
    i_pre = _normal(rng, (B, NH, S), w.i_mu, w.i_sd)
    f_pre = _normal(rng, (B, NH, S), w.f_mu, w.f_sd)
    o_pre = _normal(rng, (B, NH, S, dv))
    if w.spike_frac > 0.0:
        n_spikes = int(math.floor(w.spike_frac * B * NH * S))
        pos = rng.permutation(B * NH * S)[:n_spikes]
        i_pre.reshape(-1)[pos] = np.float32(w.spike_value)
    if w.scale_k:
        k *= np.float32(1.0 / math.sqrt(dqk))
    if w.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return dict(q=q, k=k, v=v, i_pre=i_pre, f_pre=f_pre, o_pre=o_pre)


def bwd_dh(w: Workload, seed: int | None = None, B: int | None = None, NH: int | None = None,
           S: int | None = None, dv: int | None = None) -> np.ndarray:
    """Gradient with respect to h for a backward: N(0,1) [B,NH,S,dv] float32, bf16-rounded
    for bf16 workloads (generator seeded with seed + 2000)."""
    B = w.B if B is None else B
    NH = w.NH if NH is None else NH
    S = w.S if S is None else S
    dv = w.dv if dv is None else dv
    rng = np.random.default_rng((w.seed if seed is None else seed) + 2000)
    dh = _normal(rng, (B, NH, S, dv))
    return bf16_round(dh) if w.dtype == "bf16" else dh


def epilogue_inputs(w: Workload, seed: int | None = None, B: int | None = None, NH: int | None = None,
                    S: int | None = None, dv: int | None = None):
    """Inputs of the mLSTM block epilogue (generator seeded with seed + 3000).

    h, x, z ~ N(0,1) [B,NH,S,dv] (bf16-rounded for bf16 workloads); per-channel
    parameters [NH,dv] float32: gn_w ~ 1 + 0.1 N(0,1), gn_b ~ 0.1 N(0,1),
    skip_w ~ 1 + 0.1 N(0,1) (away from 1 and 0, so a wrong channel index shows).
    """
    B = w.B if B is None else B
    NH = w.NH if NH is None else NH
    S = w.S if S is None else S
    dv = w.dv if dv is None else dv
    rng = np.random.default_rng((w.seed if seed is None else seed) + 3000)
    h = _normal(rng, (B, NH, S, dv))
    x = _normal(rng, (B, NH, S, dv))
    z = _normal(rng, (B, NH, S, dv))
    gn_w = _normal(rng, (NH, dv), 1.0, 0.1)
    gn_b = _normal(rng, (NH, dv), 0.0, 0.1)
    skip_w = _normal(rng, (NH, dv), 1.0, 0.1)
    if w.dtype == "bf16":
        h, x, z = bf16_round(h), bf16_round(x), bf16_round(z)
    return dict(h=h, x=x, z=z, gn_w=gn_w, gn_b=gn_b, skip_w=skip_w)


def slstm_inputs(w: Workload, seed: int | None = None, B: int | None = None, NH: int | None = None,
                 S: int | None = None, dh: int | None = None):
    """Inputs of the sLSTM recurrence (generator seeded with seed + 4000).

    x_pre [B,NH,S,4,dh] float32: z~, i~, o~ ~ N(0,1), f~ ~ N(f_mu, f_sd) (forget gates
    mostly open); R [NH,4,dh,dh] ~ N(0,1)/sqrt(dh), so that R h is O(1), bf16-rounded
    for bf16 workloads.
    """
    B = w.B if B is None else B
    NH = w.NH if NH is None else NH
    S = w.S if S is None else S
    dh = w.dqk if dh is None else dh
    rng = np.random.default_rng((w.seed if seed is None else seed) + 4000)
    x = _normal(rng, (B, NH, S, 4, dh))
    x[:, :, :, 2, :] = _normal(rng, (B, NH, S, dh), w.f_mu, w.f_sd)
    R = _normal(rng, (NH, 4, dh, dh))
    R *= np.float32(1.0 / math.sqrt(dh))
    if w.dtype == "bf16":
        R = bf16_round(R)
    return dict(x_pre=x, R=R)


def step_state(w: Workload, seed: int | None = None, B: int | None = None, NH: int | None = None,
               dqk: int | None = None, dv: int | None = None):
    """Random stabilized decode state: C' ~ N(0,1)/d, n' ~ N(0,1), m ~ U(0,5), float32."""
    B = w.B if B is None else B
    NH = w.NH if NH is None else NH
    dqk = w.dqk if dqk is None else dqk
    dv = w.dv if dv is None else dv
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1000)
    C = _normal(rng, (B, NH, dv, dqk))
    C *= np.float32(1.0 / dqk)
    n = _normal(rng, (B, NH, dqk))
    m = rng.uniform(0.0, 5.0, (B, NH)).astype(np.float32)
    return dict(C=C, n=n, m=m)


def step_inputs(w: Workload, steps: int | None = None, seed: int | None = None, B: int | None = None,
                NH: int | None = None, dqk: int | None = None, dv: int | None = None):
    """Per-step inputs of ``steps`` consecutive decode steps: arrays with a leading step axis.

    q,k [T,B,NH,dqk]; v,o_pre [T,B,NH,dv]; i_pre,f_pre [T,B,NH]; i~ ~ N(0,1), f~ ~ N(3,1),
    o~ ~ N(0,1), q/k/v ~ N(0,1) rounded to bf16 for bf16 workloads.
    """
    T = w.S if steps is None else steps
    B = w.B if B is None else B
    NH = w.NH if NH is None else NH
    dqk = w.dqk if dqk is None else dqk
    dv = w.dv if dv is None else dv
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _normal(rng, (T, B, NH, dqk))
    k = _normal(rng, (T, B, NH, dqk))
    v = _normal(rng, (T, B, NH, dv))
    i_pre = _normal(rng, (T, B, NH), w.i_mu, w.i_sd)
    f_pre = _normal(rng, (T, B, NH), w.f_mu, w.f_sd)
    o_pre = _normal(rng, (T, B, NH, dv))
    if w.scale_k:
        k *= np.float32(1.0 / math.sqrt(dqk))
    if w.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return dict(q=q, k=k, v=v, i_pre=i_pre, f_pre=f_pre, o_pre=o_pre)
