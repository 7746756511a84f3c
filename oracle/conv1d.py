"""Causal depthwise conv1d state update with SiLU (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The decode step before a Mamba-2 mixer: each channel keeps its last W-1 inputs as
the conv state, stored channel-major with the time axis fastest -- the (dim,
state_len) "DS" layout of the vLLM disaggregated-serving page, section "DS Layout",
where a Nemotron-H conv state is (3072, 3) in bf16.  One step forms the window
[state, x_t], applies the channel's W taps (the last tap multiplies x_t), applies
SiLU, and shifts the window into the state.  No bias term is read.

Front-end of a Mamba-2 mixer: the conv runs over the xBC channels [x | B | C]
(H d + 2 G n of them); x gives the per-head values v, B the keys k and C the
queries q of the group.  Where the fused kernel hands those outputs on in the
ring's bf16 precision, ``round_bf16`` rounds them to nearest, ties to even.
"""
from __future__ import annotations

import numpy as np

from .rounding import round_bf16  # noqa: F401  (the fused front-end's output rounding)


def silu(x):
    return x / (1.0 + np.exp(-x))


def update(state, x, weight):
    """state [B,C,W-1], x [B,C], weight [C,W] (float64).
    Returns (out [B,C], new_state [B,C,W-1])."""
    window = np.concatenate([state, x[:, :, None]], axis=-1)       # [B,C,W]
    prods = window * weight[None, :, :]
    pre = prods[:, :, 0]
    for w in range(1, window.shape[-1]):                            # oldest tap first
        pre = pre + prods[:, :, w]
    return silu(pre), window[:, :, 1:]


def split_xbc(out, H, d, G, n):
    """Channels [x | B | C] of the conv output [Bt, H d + 2 G n] as
    v [Bt, H, d], k [Bt, G, n], q [Bt, G, n]."""
    Bt = out.shape[0]
    v = out[:, :H * d].reshape(Bt, H, d)
    k = out[:, H * d:H * d + G * n].reshape(Bt, G, n)
    q = out[:, H * d + G * n:].reshape(Bt, G, n)
    return v, k, q
