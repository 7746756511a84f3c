"""Mamba-2 single-token decode, the reference definition (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "ReplaySSM: Cache SSM Inputs, Not State", background section "memory-bound:
I/O dominates, compute starves": the recurrence

    S_t = a_t S_{t-1} + Delta_t (v_t k_t^T),      y_t = S_t q_t,      a_t = exp(A Delta_t),

with a per-head state S of shape (d, n), v in R^d, and k, q in R^n shared by the
heads of a group.  The speculative "baseline" (algorithms section, speculative
decoding) updates the state serially per draft and keeps a full snapshot of each,
restoring the snapshot of the last accepted draft.

Shapes: S [B, H, d, n]; v [B, H, d]; k, q [B, G, n]; dt, Delta, a [B, H];
A, dt_bias [H].  Head h reads the k/q of group h // (H // G).
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    """log(1 + e^x) in float64; for x > 20 written as x + log(1 + e^-x) so the
    exponential cannot overflow."""
    x = np.asarray(x, dtype=np.float64)
    big = x > 20.0
    return np.where(big, x + np.log1p(np.exp(-np.abs(x))), np.log1p(np.exp(np.minimum(x, 20.0))))


def group_of_head(H: int, G: int) -> np.ndarray:
    """Group index of every head: contiguous blocks of H // G heads."""
    assert H % G == 0
    return np.arange(H) // (H // G)


def step_size_and_decay(dt, dt_bias, A):
    """Delta = softplus(dt + dt_bias[h]) and a = exp(A[h] * Delta).

    dt is [..., H] (raw); dt_bias and A are [H].  The decay a_t = e^{A Delta_t} is
    the background section's definition; the softplus with a per-head bias is the
    usual Mamba-2 discretisation of the raw step.
    """
    dt = np.asarray(dt, np.float64)
    delta = softplus(dt + np.asarray(dt_bias, np.float64))
    a = np.exp(np.asarray(A, np.float64) * delta)
    return delta, a


def standard_step(S, v, k, q, delta, a, G):
    """One decode step of the recurrence for every request and head.

    Returns (S_t, y_t); S_t is a new array.
      S_t = a_t S_{t-1} + Delta_t v_t k_t^T ;  y_t = S_t q_t
    """
    S = np.asarray(S, np.float64)
    B, H, d, n = S.shape
    grp = group_of_head(H, G)
    kh = k[:, grp, :]                     # [B, H, n]
    qh = q[:, grp, :]
    outer = v[:, :, :, None] * kh[:, :, None, :]          # v k^T  [B, H, d, n]
    S_new = a[:, :, None, None] * S + delta[:, :, None, None] * outer
    y = np.sum(S_new * qh[:, :, None, :], axis=-1)        # S q    [B, H, d]
    return S_new, y


def run_standard(S0, steps, dt_bias, A, G):
    """Run the recurrence over a list of step inputs.

    ``steps`` is a list of dicts with float64 v [B,H,d], k, q [B,G,n] and raw
    dt [B,H].  Returns (list of y_t, list of S_t).
    """
    S = np.asarray(S0, np.float64)
    ys, Ss = [], []
    for st in steps:
        delta, a = step_size_and_decay(st["dt"], dt_bias, A)
        S, y = standard_step(S, st["v"], st["k"], st["q"], delta, a, G)
        ys.append(y)
        Ss.append(S)
    return ys, Ss


def spec_round_snapshot(S_c, drafts, dt_bias, A, G, accepted):
    """Speculative round with per-draft snapshots (the speculative baseline).

    drafts: dict with v [B,T,H,d], k, q [B,T,G,n], raw dt [B,T,H] (float64).
    Every draft position s is run serially from the committed state; y_s is read
    from the state after draft s, and the snapshot after draft s is kept.  The
    committed state becomes the snapshot after ``accepted[b]`` drafts (0 keeps
    S_c).  Returns (y [B,T,H,d], new committed state).
    """
    S = np.asarray(S_c, np.float64)
    T = drafts["v"].shape[1]
    snaps = [S]
    ys = []
    for s in range(T):
        delta, a = step_size_and_decay(drafts["dt"][:, s], dt_bias, A)
        S, y = standard_step(S, drafts["v"][:, s], drafts["k"][:, s], drafts["q"][:, s],
                             delta, a, G)
        snaps.append(S)
        ys.append(y)
    committed = np.stack([snaps[int(accepted[b])][b] for b in range(S.shape[0])])
    return np.stack(ys, axis=1), committed
