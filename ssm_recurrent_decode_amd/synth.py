"""Seeded synthetic inputs for batched single-token SSM decode.

This module only draws random tensors with the workload distributions and rounds
them to the dtypes the kernels take. It holds none of the decode method's
arithmetic, so both the GPU path and the CPU oracle can consume its output.

Conventions
-----------
* ``N(mu, s2)`` means mean ``mu`` and *variance* ``s2`` (so ``N(0, 1/n)`` has
  standard deviation ``n**-0.5``).
* bf16 tensors are returned as ``uint16`` bit patterns: the value is drawn in
  float64, rounded to float32 (round-to-nearest-even), then to bf16 by
  round-to-nearest-even on the float32 bit pattern.
* Every tensor comes from its own generator keyed by
  ``SeedSequence([seed, config_id, tensor_id, *index])`` so any step, round or
  request can be regenerated on its own.
* Per-request tensors that are large (the fp32 checkpoint state) are keyed per
  request, so a sampled subset of requests can be regenerated without the rest.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

# tensor ids used in the seed key (stable: changing them changes every input)
_T_A, _T_DTBIAS, _T_S0, _T_V, _T_K, _T_Q, _T_DT = 1, 2, 3, 4, 5, 6, 7
_T_G, _T_BETA, _T_ACCEPT = 8, 9, 10
_T_CONV_STATE, _T_CONV_W, _T_CONV_X = 11, 12, 13

BASE_SEED = 20260601


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def _gen(seed: int, cfg_id: int, tensor_id: int, *index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tensor_id, *index]))


def _normal_f32(g: np.random.Generator, shape, var: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float64) * math.sqrt(var)).astype(np.float32)


@dataclass(frozen=True)
class Shape:
    """Decode workload shape.

    batch B, nheads H, head_dim d, state_dim n, ngroups G (k/q shared by the H/G
    contiguous heads of a group), ring capacity L, draft window T (1 = plain decode).
    """
    batch: int
    nheads: int
    head_dim: int
    state_dim: int
    ngroups: int
    capacity: int
    T: int = 1

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    shape: Shape
    steps: int            # decode steps, or verify rounds for T > 1
    kind: str             # "mamba2", "mamba2_spec", "gdn_spec"
    conv_channels: int = 0
    conv_width: int = 4
    seed: int = BASE_SEED

    @property
    def cfg_seed(self) -> int:
        return self.seed + self.cfg_id


WORKLOADS = {
    0: Workload(0, "tiny Mamba-2 decode B=4 H=8 d=64 n=128 G=1 L=8, 32 steps",
                Shape(4, 8, 64, 128, 1, 8), 32, "mamba2"),
    1: Workload(1, "Nemotron-H-like SSM layer B=256 H=32 d=64 n=128 G=8 L=16, 1024 steps, conv 3072x3",
                Shape(256, 32, 64, 128, 8, 16), 1024, "mamba2", conv_channels=3072),
    2: Workload(2, "speculative verify Mamba-2 B=512 H=32 d=64 n=128 G=1 L=16 T=4, 256 rounds",
                Shape(512, 32, 64, 128, 1, 16, T=4), 256, "mamba2_spec"),
    3: Workload(3, "large SSM layer B=256 H=128 d=64 n=128 G=8, L swept 4/8/16/32, 2048 steps",
                Shape(256, 128, 64, 128, 8, 16), 2048, "mamba2"),
    4: Workload(4, "Gated DeltaNet B=256 H=32 d=128 n=128 G=32 L=16 T=4, 512 rounds",
                Shape(256, 32, 128, 128, 32, 16, T=4), 512, "gdn_spec"),
}


# ---------------------------------------------------------------- Mamba-2 layer
def mamba2_head_params(shape: Shape, seed: int, cfg_id: int, layer: int = 0):
    """Per-head A = -exp(U(0, ln 16)) and dt_bias ~ U(-4, -2), float32 [H]."""
    H = shape.nheads
    A = -np.exp(_gen(seed, cfg_id, _T_A, layer).uniform(0.0, math.log(16.0), H))
    dt_bias = _gen(seed, cfg_id, _T_DTBIAS, layer).uniform(-4.0, -2.0, H)
    return A.astype(np.float32), dt_bias.astype(np.float32)


def state0_request(shape: Shape, seed: int, cfg_id: int, b: int, layer: int = 0,
                   var: float = 0.1) -> np.ndarray:
    """Checkpoint state of one request, fp32 [H, d, n] ~ N(0, var)."""
    g = _gen(seed, cfg_id, _T_S0, layer, b)
    return _normal_f32(g, (shape.nheads, shape.head_dim, shape.state_dim), var)


def state0(shape: Shape, seed: int, cfg_id: int, layer: int = 0, var: float = 0.1,
           requests=None) -> np.ndarray:
    """Checkpoint state fp32 [len(requests) or B, H, d, n]."""
    reqs = range(shape.batch) if requests is None else requests
    out = np.empty((len(reqs), shape.nheads, shape.head_dim, shape.state_dim), np.float32)
    for i, b in enumerate(reqs):
        out[i] = state0_request(shape, seed, cfg_id, b, layer, var)
    return out


def mamba2_step_inputs(shape: Shape, seed: int, cfg_id: int, step: int, layer: int = 0):
    """One decode step (T = 1) or one verify round (T > 1).

    v ~ N(0,1) bf16, k, q ~ N(0, 1/n) bf16, dt ~ N(0,1) fp32 (raw, before
    dt_bias and softplus).  Shapes for T = 1: v [B,H,d], k/q [B,G,n], dt [B,H];
    for T > 1 a draft axis follows the batch axis: v [B,T,H,d], k/q [B,T,G,n],
    dt [B,T,H].
    """
    B, H, d, n, G, T = (shape.batch, shape.nheads, shape.head_dim, shape.state_dim,
                        shape.ngroups, shape.T)
    lead = (B,) if T == 1 else (B, T)
    v = f32_to_bf16_bits(_normal_f32(_gen(seed, cfg_id, _T_V, layer, step), lead + (H, d), 1.0))
    k = f32_to_bf16_bits(_normal_f32(_gen(seed, cfg_id, _T_K, layer, step), lead + (G, n), 1.0 / n))
    q = f32_to_bf16_bits(_normal_f32(_gen(seed, cfg_id, _T_Q, layer, step), lead + (G, n), 1.0 / n))
    dt = _normal_f32(_gen(seed, cfg_id, _T_DT, layer, step), lead + (H,), 1.0)
    return {"v": v, "k": k, "q": q, "dt": dt}


def accept_draws(seed: int, cfg_id: int, rounds: int, batch: int, T: int) -> np.ndarray:
    """Accepted draft counts, int32 [rounds, B], uniform on {0, ..., T}."""
    g = _gen(seed, cfg_id, _T_ACCEPT)
    return g.integers(0, T + 1, size=(rounds, batch), dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------- Gated DeltaNet
def gdn_round_inputs(shape: Shape, seed: int, cfg_id: int, rnd: int, layer: int = 0):
    """One verify round of Gated DeltaNet drafts (or one step when T = 1).

    v ~ N(0,1) bf16 [B,T,H,d]; k ~ N(0,1/n) then L2-normalised (in float64,
    before rounding) bf16 [B,T,G,n]; q ~ N(0,1/n) bf16 [B,T,G,n];
    beta = sigmoid(N(0,1)) fp32 [B,T,H]; g = -softplus(N(0,1)) fp32 [B,T,H].
    The gate and beta are handed to the kernels already activated.
    """
    B, H, d, n, G, T = (shape.batch, shape.nheads, shape.head_dim, shape.state_dim,
                        shape.ngroups, shape.T)
    v = f32_to_bf16_bits(_normal_f32(_gen(seed, cfg_id, _T_V, layer, rnd), (B, T, H, d), 1.0))
    kr = _gen(seed, cfg_id, _T_K, layer, rnd).standard_normal((B, T, G, n)) / math.sqrt(n)
    kr = kr / np.sqrt(np.sum(kr * kr, axis=-1, keepdims=True))
    k = f32_to_bf16_bits(kr.astype(np.float32))
    q = f32_to_bf16_bits(_normal_f32(_gen(seed, cfg_id, _T_Q, layer, rnd), (B, T, G, n), 1.0 / n))
    zb = _gen(seed, cfg_id, _T_BETA, layer, rnd).standard_normal((B, T, H))
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    zg = _gen(seed, cfg_id, _T_G, layer, rnd).standard_normal((B, T, H))
    g = (-np.logaddexp(0.0, zg)).astype(np.float32)
    return {"v": v, "k": k, "q": q, "g": g, "beta": beta}


# ---------------------------------------------------------------- causal conv1d
def conv_layer(batch: int, channels: int, width: int, seed: int, cfg_id: int, layer: int = 0):
    """Conv state bf16 [B, C, W-1] ~ N(0,1) (channel-major, state_len fastest)
    and weights bf16 [C, W] ~ N(0, 0.5)."""
    st = _normal_f32(_gen(seed, cfg_id, _T_CONV_STATE, layer), (batch, channels, width - 1), 1.0)
    w = _normal_f32(_gen(seed, cfg_id, _T_CONV_W, layer), (channels, width), 0.5)
    return f32_to_bf16_bits(st), f32_to_bf16_bits(w)


def conv_step_input(batch: int, channels: int, seed: int, cfg_id: int, step: int, layer: int = 0):
    """New conv input x bf16 [B, C] ~ N(0,1)."""
    return f32_to_bf16_bits(_normal_f32(_gen(seed, cfg_id, _T_CONV_X, layer, step),
                                        (batch, channels), 1.0))
