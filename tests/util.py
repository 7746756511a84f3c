"""Helpers shared by the tests: error metrics and small float64 input builders.

Nothing here computes any part of the decode method."""
from __future__ import annotations

import numpy as np


def rel_err(got, ref) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)) over the whole tensor.

    Elementwise relative error, floored by the tensor's RMS so entries that are
    near zero do not blow up the ratio."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0.0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))


def norm_err(got, ref) -> float:
    """max |g - r| / max |r| (normwise)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    m = float(np.max(np.abs(r))) if r.size else 0.0
    return float(np.max(np.abs(g - r))) / (m if m > 0 else 1.0)


def tiny_mamba2(rng, B, H, d, n, G, steps, T=None, s0_scale=1.0, dt_bias=None, A=None):
    """Random float64 inputs for oracle pins (not bf16-rounded)."""
    A = -np.exp(rng.uniform(0.0, np.log(16.0), H)) if A is None else np.asarray(A, np.float64)
    dt_bias = rng.uniform(-4.0, -2.0, H) if dt_bias is None else np.asarray(dt_bias, np.float64)
    S0 = rng.standard_normal((B, H, d, n)) * s0_scale
    lead = (B,) if T is None else (B, T)
    seq = []
    for _ in range(steps):
        seq.append({
            "v": rng.standard_normal(lead + (H, d)),
            "k": rng.standard_normal(lead + (G, n)) / np.sqrt(n),
            "q": rng.standard_normal(lead + (G, n)) / np.sqrt(n),
            "dt": rng.standard_normal(lead + (H,)),
        })
    return S0, seq, dt_bias, A


def tiny_gdn(rng, B, H, d, n, G, steps, T=None, s0_scale=1.0):
    S0 = rng.standard_normal((B, H, d, n)) * s0_scale
    lead = (B,) if T is None else (B, T)
    seq = []
    for _ in range(steps):
        k = rng.standard_normal(lead + (G, n))
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
        seq.append({
            "v": rng.standard_normal(lead + (H, d)),
            "k": k,
            "q": rng.standard_normal(lead + (G, n)) / np.sqrt(n),
            "g": -np.logaddexp(0.0, rng.standard_normal(lead + (H,))),
            "beta": 1.0 / (1.0 + np.exp(-rng.standard_normal(lead + (H,)))),
        })
    return S0, seq
