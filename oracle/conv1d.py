"""Causal depthwise conv1d state update with SiLU (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The decode step before a Mamba-2 mixer: each channel keeps its last W-1 inputs as
the conv state, stored channel-major with the time axis fastest -- the (dim,
state_len) "DS" layout of the vLLM disaggregated-serving page, section "DS Layout",
where a Nemotron-H conv state is (3072, 3) in bf16.  One step forms the window
[state, x_t], applies the channel's W taps (the last tap multiplies x_t), applies
SiLU, and shifts the window into the state.  No bias term is read.
"""
from __future__ import annotations

import numpy as np


def silu(x):
    return x / (1.0 + np.exp(-x))


def update(state, x, weight):
    """state [B,C,W-1], x [B,C], weight [C,W] (float64).
    Returns (out [B,C], new_state [B,C,W-1])."""
    window = np.concatenate([state, x[:, :, None]], axis=-1)       # [B,C,W]
    pre = np.sum(window * weight[None, :, :], axis=-1)
    return silu(pre), window[:, :, 1:]
