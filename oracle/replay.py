"""ReplaySSM decode bookkeeping for Mamba-2, written out on its own (float64, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

This is a second, separate plain implementation of the decode path, kept to pin the
ring bookkeeping against the definition in ``oracle.mamba2``.  It follows
"ReplaySSM: Cache SSM Inputs, Not State":

* method, core idea: keep a checkpoint S_0 and a ring of the most recent inputs
  instead of writing the state back every step; fold the ring into S_0 ("flush")
  only when it fills;
* method, output-only decode: between flushes
      y_t = abar_t (S_0 q_t) + sum_{j=1}^{t} s_{j,t} v_j (k_j^T q_t),
  read by inner products, never materialising the state;
* algorithms, Mamba-2 standard decode: append (v, Delta, k), compute the decay
  weights, read y, flush if the buffer is full;
* algorithms, speculative decoding: append the T drafts; y for draft s uses the
  checkpoint and every entry up to its own position p_s; a flush folds only the
  committed entries; flush early when h + 2T > L;
* kernel design, ring buffer: entries are addressed modulo L from a head pointer,
  so rollback of rejected drafts only moves a pointer.

Readings (the page defines abar and s_{j,t} only through the unrolled history form
of the core-idea section): with entries numbered 1..c in arrival order since the
checkpoint,
    abar = prod_{i=1}^{c} a_i,        s_j = Delta_j * prod_{j<i<=c} a_i .
"""
from __future__ import annotations

import numpy as np

from .mamba2 import group_of_head, step_size_and_decay


class _Entry:
    """One cached input: v [H,d], k [G,n], Delta [H], a [H]."""
    __slots__ = ("v", "k", "delta", "a")

    def __init__(self, v, k, delta, a):
        self.v, self.k, self.delta, self.a = v, k, delta, a


class ReplayRequest:
    """Decode memory of one request: checkpoint S_0 [H,d,n], ring of capacity L,
    head (slot of the oldest cached entry), count (committed entries since the
    checkpoint) and pending (uncommitted draft entries after them)."""

    def __init__(self, S0, L: int, G: int):
        self.S0 = np.array(S0, dtype=np.float64)
        self.H, self.d, self.n = self.S0.shape
        self.L, self.G = L, G
        self.grp = group_of_head(self.H, G)
        self.ring = [None] * L
        self.head = 0
        self.count = 0
        self.pending = 0

    # -- helpers -------------------------------------------------------------
    def _logical(self, num):
        """The first ``num`` cached entries in arrival order."""
        return [self.ring[(self.head + j) % self.L] for j in range(num)]

    @staticmethod
    def _weights(entries, H):
        """abar = prod_i a_i and s_j = Delta_j prod_{i>j} a_i, as explicit products."""
        abar = np.ones(H)
        for e in entries:
            abar = abar * e.a
        s = []
        for j in range(len(entries)):
            w = np.array(entries[j].delta, dtype=np.float64)
            for i in range(j + 1, len(entries)):
                w = w * entries[i].a
            s.append(w)
        return abar, s

    def _read(self, q, entries):
        """Output-only route: abar (S_0 q) + sum_j s_j (k_j . q) v_j  -> [H, d]."""
        abar, s = self._weights(entries, self.H)
        qh = q[self.grp]                                       # [H, n]
        y = abar[:, None] * np.sum(self.S0 * qh[:, None, :], axis=-1)
        for j, e in enumerate(entries):
            kq = np.sum(e.k[self.grp] * qh, axis=-1)           # k_j^T q  [H]
            y = y + (s[j] * kq)[:, None] * e.v
        return y

    def _fold(self, entries):
        """Flush: S_0 <- abar S_0 + sum_j s_j v_j k_j^T  (state-and-output route)."""
        abar, s = self._weights(entries, self.H)
        S = abar[:, None, None] * self.S0
        for j, e in enumerate(entries):
            S = S + s[j][:, None, None] * (e.v[:, :, None] * e.k[self.grp][:, None, :])
        self.S0 = S

    # -- standard decode -----------------------------------------------------
    def decode_step(self, v, k, q, delta, a):
        """Append, read y, flush when the ring is full.  Returns (y [H,d], flushed).

        v [H,d], k, q [G,n], delta, a [H] are this request's float64 inputs.
        The flush happens on the step whose append fills the ring, and that step's
        y equals the read of the folded state."""
        assert self.pending == 0 and 0 <= self.count < self.L
        self.ring[(self.head + self.count) % self.L] = _Entry(v, k, delta, a)
        self.count += 1
        entries = self._logical(self.count)
        y = self._read(q, entries)
        flushed = False
        if self.count == self.L:
            self._fold(entries)
            self.head = (self.head + self.count) % self.L
            self.count = 0
            flushed = True
        return y, flushed

    def flush(self):
        """Explicit flush of the committed entries (pending drafts stay cached)."""
        if self.count == 0:
            return False
        self._fold(self._logical(self.count))
        self.head = (self.head + self.count) % self.L
        self.count = 0
        return True

    # -- speculative decode --------------------------------------------------
    def verify_round(self, v, k, q, delta, a):
        """Verify T drafts: v [T,H,d], k, q [T,G,n], delta, a [T,H].

        Drafts go to the slots after the committed entries; draft s reads the
        checkpoint and the entries up to its own position c + s + 1.  If
        c + 2T > L the c committed entries are folded into S_0 (drafts are never
        folded).  Returns (y [T,H,d], flushed)."""
        T = v.shape[0]
        c = self.count
        assert self.pending == 0 and c + T <= self.L, "window would be truncated"
        for s in range(T):
            self.ring[(self.head + c + s) % self.L] = _Entry(v[s], k[s], delta[s], a[s])
        self.pending = T
        ys = []
        for s in range(T):
            ys.append(self._read(q[s], self._logical(c + s + 1)))
        flushed = False
        if c + 2 * T > self.L:
            if c > 0:
                self._fold(self._logical(c))
            self.head = (self.head + c) % self.L
            self.count = 0
            flushed = True
        return np.stack(ys), flushed

    def commit(self, accepted: int):
        """Rollback/commit: keep the first ``accepted`` drafts; drop the rest by
        leaving them beyond ``count``."""
        assert 0 <= accepted <= self.pending
        self.count += accepted
        self.pending = 0


def run_standard(S0, steps, dt_bias, A, L, G):
    """Drive ReplayRequest over a step sequence for each request.

    S0 [B,H,d,n]; steps is a list of dicts with float64 v [B,H,d], k, q [B,G,n]
    and raw dt [B,H].  Returns (ys [steps][B,H,d], flush flags [steps][B] bool,
    final request objects)."""
    B = S0.shape[0]
    reqs = [ReplayRequest(S0[b], L, G) for b in range(B)]
    ys, fl = [], []
    for st in steps:
        delta, a = step_size_and_decay(st["dt"], dt_bias, A)
        yb, fb = [], []
        for b, r in enumerate(reqs):
            y, f = r.decode_step(st["v"][b], st["k"][b], st["q"][b], delta[b], a[b])
            yb.append(y)
            fb.append(f)
        ys.append(np.stack(yb))
        fl.append(np.array(fb))
    return ys, fl, reqs


def run_spec(S0, rounds, dt_bias, A, L, G, accepted):
    """Drive ReplayRequest over verify rounds with the given acceptance.

    rounds: list of dicts with float64 v [B,T,H,d], k, q [B,T,G,n], raw dt [B,T,H];
    accepted: int [R, B].  Returns (ys [R][B,T,H,d], flush flags [R][B] bool,
    per-round start counts [R][B] int, final request objects)."""
    B = S0.shape[0]
    reqs = [ReplayRequest(S0[b], L, G) for b in range(B)]
    ys, fl, starts = [], [], []
    for r, rd in enumerate(rounds):
        delta, a = step_size_and_decay(rd["dt"], dt_bias, A)
        yb, fb, cb = [], [], []
        for b, q in enumerate(reqs):
            cb.append(q.count)
            y, f = q.verify_round(rd["v"][b], rd["k"][b], rd["q"][b], delta[b], a[b])
            q.commit(int(accepted[r][b]))
            yb.append(y)
            fb.append(f)
        ys.append(np.stack(yb))
        fl.append(np.array(fb))
        starts.append(np.array(cb))
    return ys, fl, starts, reqs


def pointer_schedule_standard(L: int, steps: int, head0: int = 0, count0: int = 0):
    """Integer bookkeeping of standard decode alone: per step (head, count,
    flushed) after the call.  Append adds one entry; the step that fills the ring
    folds all L entries and moves head past them."""
    head, count = head0, count0
    out = []
    for _ in range(steps):
        count += 1
        flushed = count == L
        if flushed:
            head = (head + count) % L
            count = 0
        out.append((head, count, flushed))
    return out


def pointer_schedule_spec(L: int, T: int, accepted):
    """Integer bookkeeping of speculative rounds alone, for one request:
    per round (count at round start, flushed, head after verify, count after
    verify, count after commit).  The verify folds the committed entries when
    c + 2T > L; the commit keeps ``accepted[r]`` drafts."""
    head, count = 0, 0
    out = []
    for a in accepted:
        c = count
        flushed = c + 2 * T > L
        if flushed:
            head = (head + c) % L
            count = 0
        after_verify = (head, count)
        count += int(a)
        out.append((c, flushed, after_verify[0], after_verify[1], count))
    return out
