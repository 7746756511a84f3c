"""Decode-state memory per request and the largest batch a fixed HBM budget holds.

"ReplaySSM: Cache SSM Inputs, Not State", results ("higher maximum
concurrency"): at a fixed HBM budget the speculative baseline's per-draft state
snapshots cut the largest decode batch about fourfold; ReplaySSM keeps one state
plus a ring of small input vectors and recovers most of that capacity.  Per SSM
layer and request, with this library's layouts:

* standard decode:  one fp32 state, 4 H d n bytes;
* snapshot route:   T + 1 state slots (the committed one and one per draft) and
                    the int32 slot index;
* ReplaySSM:        the checkpoint plus the ring -- v bf16 (GDN: u fp32) [H, L, d],
                    k bf16 [G, L, n] and the per-head ring records
                    [H, RSSM_META_WORDS(L)] fp32 (the same sizes rssm_ring_sizes
                    reports), plus the 4-byte error word shared by the batch.

Host arithmetic only; nothing here runs on the device.
"""
from __future__ import annotations

F32, BF16 = 4, 2


def meta_words(L: int) -> int:
    return 32 if L + 3 <= 32 else 64


def state_bytes(H: int, d: int, n: int) -> int:
    return F32 * H * d * n


def ring_bytes_per_request(H: int, d: int, n: int, G: int, L: int, gdn: bool = False) -> int:
    """v (or u) + k + records of one request's ring."""
    return H * L * d * (F32 if gdn else BF16) + G * L * n * BF16 + H * meta_words(L) * F32


def bytes_per_request(route: str, H: int, d: int, n: int, G: int, L: int = 16, T: int = 4,
                      gdn: bool = False) -> int:
    """SSM decode memory of one request in one layer for route 'standard',
    'snapshot' (T + 1 slots) or 'replay' (ring capacity L)."""
    if route == "standard":
        return state_bytes(H, d, n)
    if route == "snapshot":
        return (T + 1) * state_bytes(H, d, n) + 4
    if route == "replay":
        return state_bytes(H, d, n) + ring_bytes_per_request(H, d, n, G, L, gdn)
    raise ValueError(f"unknown route {route!r}")


def max_batch(budget_bytes: int, per_request_bytes: int, layers: int = 1, shared_bytes: int = 0) -> int:
    """Largest number of requests whose decode state fits the budget."""
    room = budget_bytes - shared_bytes
    return max(0, room // (per_request_bytes * layers))


def concurrency_table(H: int, d: int, n: int, G: int, L: int, T: int, gdn: bool,
                      budget_bytes: int) -> dict:
    """Bytes per request and the largest batch per route for one layer's state in
    the budget (for a stack of m SSM layers divide the batches by m)."""
    per = {r: bytes_per_request(r, H, d, n, G, L, T, gdn) for r in ("standard", "snapshot", "replay")}
    mb = {r: max_batch(budget_bytes, b, shared_bytes=4 if r == "replay" else 0) for r, b in per.items()}
    return {"bytes_per_request": per, "max_batch": mb,
            "replay_over_snapshot": round(mb["replay"] / mb["snapshot"], 3),
            "snapshot_over_standard": round(mb["snapshot"] / mb["standard"], 3)}
