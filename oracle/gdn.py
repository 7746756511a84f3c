"""Gated DeltaNet decode, reference implementations (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources, all on "ReplaySSM: Cache SSM Inputs, Not State":

* background section: the delta-rule recurrence
      S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   y_t = S_t q_t,
  where (I - beta k k^T) is the Householder term;
* appendix, GDN standard decode: ReplaySSM caches the correction
      u_t = beta_t (v_t - alpha_t S_{t-1} k_t),   alpha_t = e^{g_t},
  which turns the update into S_t = alpha_t S_{t-1} + u_t k_t^T, the same history
  form as Mamba-2; the state-and-output route rebuilds
      S_h = (prod_j alpha_j) S_0 + sum_j (prod_{i>j} alpha_i) u_j k_j^T ;
* appendix, GDN speculative decoding: unrolling the window gives
      u_s = R_s - sum_{s'<s} A_{s,s'} u_{s'},
  one strictly lower-triangular T x T solve for all T corrections.

Reading: the appendix writes the correction without the gate (u = beta(v - S k));
with the gate of the background recurrence it is u = beta(v - alpha S k), which is
also the form the appendix's own state-and-output route uses.  The speculative
semantics (snapshot per draft, commit the snapshot of the last accepted draft)
match the Mamba-2 baseline.

Shapes: S [B,H,d,n]; v [B,H,d]; k, q [B,G,n]; g, beta [B,H].
"""
from __future__ import annotations

import numpy as np

from .mamba2 import group_of_head
from .rounding import round_bf16


def householder_step(S, v, k, q, g, beta, G):
    """One step of the delta rule, written with the Householder term:
    S_t = e^{g} S (I - beta k k^T) + beta v k^T, using S (I - beta k k^T) =
    S - beta (S k) k^T.  Returns (S_t, y_t)."""
    S = np.asarray(S, np.float64)
    B, H, d, n = S.shape
    grp = group_of_head(H, G)
    kh, qh = k[:, grp, :], q[:, grp, :]
    alpha = np.exp(g)
    Sk = np.sum(S * kh[:, :, None, :], axis=-1)                       # [B,H,d]
    erased = S - beta[:, :, None, None] * (Sk[:, :, :, None] * kh[:, :, None, :])
    S_new = alpha[:, :, None, None] * erased + beta[:, :, None, None] * (
        v[:, :, :, None] * kh[:, :, None, :])
    y = np.sum(S_new * qh[:, :, None, :], axis=-1)
    return S_new, y


def spec_round_snapshot(S_c, drafts, G, accepted):
    """Speculative round with per-draft snapshots of the delta-rule state.

    drafts: v [B,T,H,d], k, q [B,T,G,n], g, beta [B,T,H] (float64).
    Returns (y [B,T,H,d], committed state after ``accepted[b]`` drafts)."""
    S = np.asarray(S_c, np.float64)
    T = drafts["v"].shape[1]
    snaps, ys = [S], []
    for s in range(T):
        S, y = householder_step(S, drafts["v"][:, s], drafts["k"][:, s], drafts["q"][:, s],
                                drafts["g"][:, s], drafts["beta"][:, s], G)
        snaps.append(S)
        ys.append(y)
    committed = np.stack([snaps[int(accepted[b])][b] for b in range(S.shape[0])])
    return np.stack(ys, axis=1), committed


class _Entry:
    """One cached GDN input: correction u [H,d], key k [G,n], decay alpha [H]."""
    __slots__ = ("u", "k", "alpha")

    def __init__(self, u, k, alpha):
        self.u, self.k, self.alpha = u, k, alpha


class GDNReplayRequest:
    """ReplaySSM memory of one GDN request: checkpoint S_0 [H,d,n], ring of
    (u, k, alpha) with capacity L, head, count (committed), pending (drafts)."""

    def __init__(self, S0, L: int, G: int, u_bf16: bool = False):
        """u_bf16: the ring keeps the corrections in bf16 -- each u is rounded
        when it is cached; the outputs of the step that computes it use it
        unrounded."""
        self.u_bf16 = u_bf16
        self.S0 = np.array(S0, dtype=np.float64)
        self.H, self.d, self.n = self.S0.shape
        self.L, self.G = L, G
        self.grp = group_of_head(self.H, G)
        self.ring = [None] * L
        self.head = self.count = self.pending = 0

    def _logical(self, num):
        return [self.ring[(self.head + j) % self.L] for j in range(num)]

    def rebuilt_state(self, entries):
        """State-and-output route: S_h = (prod_j alpha_j) S_0 + sum_j (prod_{i>j} alpha_i) u_j k_j^T,
        with the products written out."""
        S = np.array(self.S0)
        for e in entries:                       # S <- alpha S + u k^T, oldest first
            S = e.alpha[:, None, None] * S + e.u[:, :, None] * e.k[self.grp][:, None, :]
        return S

    def rebuilt_state_closed(self, entries):
        """The same S_h from the closed sum (explicit product of the later decays)."""
        c = len(entries)
        abar = np.ones(self.H)
        for e in entries:
            abar = abar * e.alpha
        S = abar[:, None, None] * self.S0
        for j in range(c):
            w = np.ones(self.H)
            for i in range(j + 1, c):
                w = w * entries[i].alpha
            S = S + w[:, None, None] * (entries[j].u[:, :, None] * entries[j].k[self.grp][:, None, :])
        return S

    def decode_step(self, v, k, q, g, beta):
        """Standard decode (T = 1): correction from the rebuilt state, append
        (u, k, alpha), read y; flush when the ring is full.  Returns (y, flushed)."""
        assert self.pending == 0 and 0 <= self.count < self.L
        S_h = self.rebuilt_state_closed(self._logical(self.count))
        alpha = np.exp(g)
        kh, qh = k[self.grp], q[self.grp]
        u = beta[:, None] * (v - alpha[:, None] * np.sum(S_h * kh[:, None, :], axis=-1))
        y = alpha[:, None] * np.sum(S_h * qh[:, None, :], axis=-1) + u * np.sum(kh * qh, axis=-1)[:, None]
        self.ring[(self.head + self.count) % self.L] = _Entry(self._cached(u), k, alpha)
        self.count += 1
        flushed = False
        if self.count == self.L:
            self.S0 = self.rebuilt_state_closed(self._logical(self.count))
            self.head = (self.head + self.count) % self.L
            self.count = 0
            flushed = True
        return y, flushed

    def verify_round(self, v, k, q, g, beta):
        """Verify T drafts serially from the rebuilt committed state.

        v [T,H,d], k, q [T,G,n], g, beta [T,H].  For each draft s:
        u_s = beta_s (v_s - alpha_s S k_s); S <- alpha_s S + u_s k_s^T; y_s = S q_s;
        (u_s, k_s, alpha_s) is cached after the committed entries.  If c + 2T > L
        the committed state S_h becomes the new checkpoint.  Returns
        (y [T,H,d], u [T,H,d], flushed)."""
        T = v.shape[0]
        c = self.count
        assert self.pending == 0 and c + T <= self.L
        S_h = self.rebuilt_state_closed(self._logical(c))
        S = S_h
        ys, us = [], []
        for s in range(T):
            alpha = np.exp(g[s])
            kh, qh = k[s][self.grp], q[s][self.grp]
            u = beta[s][:, None] * (v[s] - alpha[:, None] * np.sum(S * kh[:, None, :], axis=-1))
            S = alpha[:, None, None] * S + u[:, :, None] * kh[:, None, :]
            ys.append(np.sum(S * qh[:, None, :], axis=-1))
            us.append(u)
            self.ring[(self.head + c + s) % self.L] = _Entry(self._cached(u), k[s], alpha)
        self.pending = T
        flushed = False
        if c + 2 * T > self.L:
            self.S0 = S_h
            self.head = (self.head + c) % self.L
            self.count = 0
            flushed = True
        return np.stack(ys), np.stack(us), flushed

    def _cached(self, u):
        return round_bf16(u) if self.u_bf16 else u

    def flush(self):
        if self.count == 0:
            return False
        self.S0 = self.rebuilt_state_closed(self._logical(self.count))
        self.head = (self.head + self.count) % self.L
        self.count = 0
        return True

    def commit(self, accepted: int):
        assert 0 <= accepted <= self.pending
        self.count += accepted
        self.pending = 0


def window_decays(alpha):
    """gamma_s = prod_{i<=s} alpha_i and ratio[s, s'] = prod_{s'<i<=s} alpha_i
    (s' <= s) for one head's window alpha [T], as explicit products."""
    T = len(alpha)
    gamma = np.ones(T)
    ratio = np.zeros((T, T))
    for s in range(T):
        for i in range(s + 1):
            gamma[s] *= alpha[i]
        for sp in range(s + 1):
            r = 1.0
            for i in range(sp + 1, s + 1):
                r *= alpha[i]
            ratio[s, sp] = r
    return gamma, ratio


def chunkwise_window(S_h, v, k, q, g, beta):
    """All T corrections of one head's draft window at once.

    S_h [d,n] committed state; v [T,d]; k, q [T,n]; g, beta [T].
      R_s      = beta_s (v_s - gamma_s S_h k_s)
      A[s,s']  = beta_s (gamma_s / gamma_s') (k_s . k_s')      for s' < s
      (I + A) U = R  by forward substitution:  u_s = R_s - sum_{s'<s} A[s,s'] u_s'
      y_s      = gamma_s S_h q_s + sum_{s'<=s} (gamma_s / gamma_s') (k_s' . q_s) u_s'
    Returns (U [T,d], y [T,d], A [T,T], R [T,d])."""
    T, d = v.shape
    alpha = np.exp(g)
    gamma, ratio = window_decays(alpha)
    R = np.stack([beta[s] * (v[s] - gamma[s] * (S_h @ k[s])) for s in range(T)])
    A = np.zeros((T, T))
    for s in range(T):
        for sp in range(s):
            A[s, sp] = beta[s] * ratio[s, sp] * np.dot(k[s], k[sp])
    U = np.zeros((T, d))
    for s in range(T):
        acc = np.array(R[s])
        for sp in range(s):
            acc = acc - A[s, sp] * U[sp]
        U[s] = acc
    Y = np.zeros((T, d))
    for s in range(T):
        y = gamma[s] * (S_h @ q[s])
        for sp in range(s + 1):
            y = y + ratio[s, sp] * np.dot(k[sp], q[s]) * U[sp]
        Y[s] = y
    return U, Y, A, R
