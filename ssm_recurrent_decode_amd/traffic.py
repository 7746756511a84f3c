"""Algorithmic HBM bytes of each decode kernel launch (the minimum traffic the
operation needs, every byte counted once), for roofline reporting.

The per-head model follows the traffic paragraph of "ReplaySSM: Cache SSM Inputs,
Not State" (method, "three advantages"): the baseline moves 8dn bytes of state
plus the step inputs; ReplaySSM with h cached entries moves 4dn bytes of
checkpoint, the h cached (v, Delta, k) entries, the current inputs and the new
entry.  Here it is counted with this library's dtypes -- fp32 state, bf16 v/k/q,
fp32 step size and decay in the ring, fp32 y, fp32 GDN corrections -- and with k/q
counted once per group (they are shared by the heads of a group).
"""
from __future__ import annotations

F32, BF16 = 4, 2
PTR = 8  # one packed pointer word per request, read and written once


def standard_step(B, H, d, n, G) -> int:
    """ssm_decode_step: state read + write, v, k, q, dt in, y out, per-head params."""
    return B * (2 * F32 * H * d * n + BF16 * H * d + 2 * BF16 * G * n + F32 * H + F32 * H * d) \
        + 2 * F32 * H


def replay_slot(H, d, n, G) -> int:
    """Bytes of one cached entry of one request: v (bf16, all heads), k (bf16, per
    group), step size (fp32 per head; the decay exp(A Delta) is recomputed)."""
    return BF16 * H * d + BF16 * G * n + F32 * H


def replay_append(B, H, d, n, G, h, flush: bool) -> int:
    """replay_append_decode with h entries cached before the call.  A flush step
    writes the checkpoint back instead of caching the new entry."""
    per_req = (F32 * H * d * n                       # checkpoint read
               + h * replay_slot(H, d, n, G)         # cached entries read
               + BF16 * H * d + 2 * BF16 * G * n + F32 * H   # v, k, q, dt in
               + F32 * H * d                         # y out
               + 2 * PTR)                            # pointer word read + write
    per_req += F32 * H * d * n if flush else replay_slot(H, d, n, G)
    return B * per_req + 2 * F32 * H


def replay_append_conv(B, H, d, n, G, h, flush: bool, W: int = 4) -> int:
    """replay_append_decode_conv: as replay_append, with the conv state of the
    C = H d + 2 G n xBC channels read and written (bf16, W - 1 per channel) and
    the taps read once; the token's xBC (2C bytes) replaces the v, k, q inputs,
    which are the same bytes."""
    C = H * d + 2 * G * n
    return replay_append(B, H, d, n, G, h, flush) + B * C * 2 * BF16 * (W - 1) + C * W * BF16


def replay_verify(B, H, d, n, G, T, c, flush: bool, y_bytes: int = F32) -> int:
    """replay_verify_T with c committed entries: checkpoint read, c cached entries,
    T drafts in, T outputs (fp32, or bf16 with y_bytes = 2), T new entries
    cached, checkpoint write on a flush."""
    per_req = (F32 * H * d * n + c * replay_slot(H, d, n, G)
               + T * (BF16 * H * d + 2 * BF16 * G * n + F32 * H)
               + T * y_bytes * H * d + T * replay_slot(H, d, n, G) + 2 * PTR)
    if flush:
        per_req += F32 * H * d * n
    return B * per_req + 2 * F32 * H


def replay_flush(B, H, d, n, G, c) -> int:
    """Explicit flush of c committed entries: checkpoint read and write, the c
    cached entries, the heads' A, the pointer word read and written."""
    return B * (2 * F32 * H * d * n + c * replay_slot(H, d, n, G) + F32 * H + 2 * PTR)


def gdn_flush(B, H, d, n, G, c) -> int:
    return B * (2 * F32 * H * d * n + c * gdn_slot(H, d, n, G) + 2 * PTR)


def gdn_slot(H, d, n, G, u_bytes: int = F32) -> int:
    """One cached GDN entry: u (fp32, or bf16 with u_bytes = 2), k (bf16 per
    group), alpha (fp32)."""
    return u_bytes * H * d + BF16 * G * n + F32 * H


def gdn_verify(B, H, d, n, G, T, c, flush: bool, y_bytes: int = F32, u_bytes: int = F32) -> int:
    per_req = (F32 * H * d * n + c * gdn_slot(H, d, n, G, u_bytes)
               + T * (BF16 * H * d + 2 * BF16 * G * n + 2 * F32 * H)
               + T * y_bytes * H * d + T * gdn_slot(H, d, n, G, u_bytes) + 2 * PTR)
    if flush:
        per_req += F32 * H * d * n
    return B * per_req


def gdn_append(B, H, d, n, G, h, flush: bool) -> int:
    """gdn_replay_append_decode with h entries cached before the call: checkpoint
    read, the h cached (u, k, alpha) entries, the token's inputs, y, the pointer
    word; the new entry cached, or the checkpoint written back on a flush step."""
    per_req = (F32 * H * d * n + h * gdn_slot(H, d, n, G)
               + BF16 * H * d + 2 * BF16 * G * n + 2 * F32 * H + F32 * H * d + 2 * PTR)
    per_req += F32 * H * d * n if flush else gdn_slot(H, d, n, G)
    return B * per_req


def gdn_standard_step(B, H, d, n, G) -> int:
    return B * (2 * F32 * H * d * n + BF16 * H * d + 2 * BF16 * G * n + 2 * F32 * H + F32 * H * d)


def snapshot_verify(B, H, d, n, G, T, gdn: bool = False) -> int:
    """ssm_snapshot_verify_T / gdn_snapshot_verify_T: the committed state read once,
    T full snapshots written, T drafts in (Mamba-2: dt; GDN: g and beta), T outputs,
    the slot index read; per-head A and dt_bias for Mamba-2."""
    scal = (2 if gdn else 1) * F32 * H
    per_req = (F32 * H * d * n + T * F32 * H * d * n
               + T * (BF16 * H * d + 2 * BF16 * G * n + scal) + T * F32 * H * d + 4)
    return B * per_req + (0 if gdn else 2 * F32 * H)


def conv1d(B, C, W) -> int:
    """conv state read + write (bf16), x in (bf16), out (fp32), taps (bf16, shared)."""
    return B * C * (2 * BF16 * (W - 1) + BF16 + F32) + C * W * BF16


def pages_traffic_per_head(d, n, h=None) -> int:
    """The page's per-head formula, with 2 bytes per vector element and scalar:
    baseline 8dn + 2(d + 2n + 1); ReplaySSM 4dn + 2h(d + n + 1) + 2(d + 2n + 1)
    + 2(d + n + 1)."""
    if h is None:
        return 8 * d * n + 2 * (d + 2 * n + 1)
    return 4 * d * n + 2 * h * (d + n + 1) + 2 * (d + 2 * n + 1) + 2 * (d + n + 1)
