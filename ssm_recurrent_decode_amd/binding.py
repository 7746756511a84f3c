"""Thin PyTorch binding of the C ABI: the same entry-point names, tensors instead of
raw pointers.  Every function only checks dtypes, shapes, contiguity and device,
then passes data pointers and the current HIP stream to the library; all compute
happens in the HIP kernels.  Non-zero return codes raise RuntimeError.

bf16 arguments may be torch.bfloat16 tensors or int16/uint16 tensors holding the
bit patterns.  PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import dataclasses
from dataclasses import dataclass

import torch

from . import _lib

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


@dataclass(frozen=True)
class Dims:
    batch: int
    nheads: int
    head_dim: int
    state_dim: int
    ngroups: int
    capacity: int = 1
    flags: int = 0   # RSSM_F_Y_BF16 | RSSM_F_U_BF16

    def c(self) -> _lib.rssm_dims:
        return _lib.rssm_dims(self.batch, self.nheads, self.head_dim, self.state_dim,
                              self.ngroups, self.capacity, self.flags)

    @property
    def y_dtypes(self):
        """Accepted dtypes of the outputs y under these flags."""
        return _BF16 if self.flags & _lib.RSSM_F_Y_BF16 else _F32


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _p(t, name, dtypes, shape, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.data_ptr() % 16 != 0:
        raise ValueError(f"{name} must be 16-byte aligned (the kernels use 16-byte vector loads)")
    return t.data_ptr()


def meta_words(L: int) -> int:
    """32-bit words of one per-head ring record (RSSM_META_WORDS)."""
    return 32 if L + 3 <= 32 else 64


def ring_head_block(H: int) -> int:
    """Heads whose ring entries of one slot are stored side by side (RSSM_RING_HEAD_BLOCK)."""
    return 4 if H % 4 == 0 else (2 if H % 2 == 0 else 1)


class Ring:
    """Device arrays of one layer's ReplaySSM ring (see rssm_ring in the header).

    Allocated zero-filled with torch on ``device``; ``gdn`` selects fp32
    corrections u instead of bf16 values v, stored [rows, H / hb, L, hb, d]
    (``entries()`` gives the [rows, H, L, d] view).  ``meta`` holds one record per
    (request, head): the packed pointer word (head in bits 0-15, count 16-31,
    pending 32-47) in words 0-1, then A and the per-slot step sizes (Mamba-2) or
    decays (GDN).  ``head``, ``count`` and ``pending`` are int32 [rows] tensors
    written by the library's rssm_ring_pointers (one per pool row), and
    ``copies_agree`` checks that every head's pointer word is the same.

    Pooled rings: ``rows`` request rows are allocated (default: the batch), and
    ``use_slots(slots)`` makes every call map batch entry b to row slots[b]
    (negative = padding entry, skipped); the checkpoint passed with it then has
    ``rows`` rows too."""

    def __init__(self, dims: Dims, gdn: bool = False, device="cuda", rows=None):
        B = dims.batch if rows is None else int(rows)
        H, G, L = dims.nheads, dims.ngroups, dims.capacity
        D, N = dims.head_dim, dims.state_dim
        self.dims, self.gdn, self.rows, self.slots = dims, gdn, B, None
        z = dict(device=device)
        u32 = gdn and not (dims.flags & _lib.RSSM_F_U_BF16)
        hb = ring_head_block(H)
        self.vu = torch.zeros((B, H // hb, L, hb, D), dtype=torch.float32 if u32 else torch.bfloat16, **z)
        self.k = torch.zeros((B, G, L, N), dtype=torch.bfloat16, **z)
        self.meta = torch.zeros((B, H, meta_words(L)), dtype=torch.float32, **z)
        self.err = torch.zeros((1,), dtype=torch.int32, **z)
        # zero-filled by torch on its current stream: finish before a call on any
        # other stream reads the records (their memory may have held another ring's)
        torch.cuda.synchronize(self.meta.device)

    @property
    def ptr(self):
        """Pointer words [B, H] (int64 view into the records)."""
        return self.meta.view(torch.int64)[:, :, 0]

    def entries(self):
        """The cached values (Mamba-2) or corrections (GDN) as a [rows, H, L, d]
        copy, head-major (``vu`` holds them in blocks of heads per slot)."""
        B, Hb, L, hb, D = self.vu.shape
        return self.vu.permute(0, 1, 3, 2, 4).reshape(B, Hb * hb, L, D)

    def pointers(self, stream=None):
        """(head, count, pending) of every pool row as int32 device tensors, from
        rssm_ring_pointers on ``stream`` (the current stream by default)."""
        out = [torch.empty((self.rows,), dtype=torch.int32, device=self.meta.device) for _ in range(3)]
        rssm_ring_pointers(dataclasses.replace(self.dims, batch=self.rows), self, *out, rows_view=True,
                           stream=stream)
        return tuple(out)

    @property
    def head(self):
        return self.pointers()[0]

    @property
    def count(self):
        return self.pointers()[1]

    @property
    def pending(self):
        return self.pointers()[2]

    def copies_agree(self) -> bool:
        w = self.ptr
        return bool(torch.all(w == w[:, :1]))

    def set_pointers(self, head=None, count=None, pending=None):
        """Overwrite pointer fields of every head's record (sequences of B ints, or
        None to keep head 0's value); each value is stored modulo 2^16 as the
        packed word holds it."""
        cur = [self.head.cpu().tolist(), self.count.cpu().tolist(), self.pending.cpu().tolist()]
        new = [list(x) if x is not None else c for x, c in zip((head, count, pending), cur)]
        words = [(h & 0xFFFF) | ((c & 0xFFFF) << 16) | ((p & 0xFFFF) << 32) for h, c, p in zip(*new)]
        col = torch.tensor(words, dtype=torch.int64).to(self.meta.device)
        self.meta.view(torch.int64)[:, :, 0] = col[:, None]
        # written by torch on its current stream: finish before a call on any
        # other stream reads the records
        torch.cuda.synchronize(self.meta.device)

    def use_slots(self, slots):
        """Map the batch entries of the following calls to pool rows (int32 device
        tensor [B]); None returns to row = batch entry."""
        if slots is not None:
            _p(slots, "slots", _I32, (int(slots.shape[0]),))
        self.slots = slots

    def c(self) -> _lib.rssm_ring:
        sp = self.slots.data_ptr() if self.slots is not None else None
        return _lib.rssm_ring(self.vu.data_ptr(), self.k.data_ptr(), self.meta.data_ptr(),
                              self.err.data_ptr(), sp, self.rows)

    def tensors(self):
        return {k: getattr(self, k) for k in ("vu", "k", "meta", "err")}


def ring_sizes(dims: Dims, gdn: bool = False):
    out = (ctypes.c_size_t * 4)()
    d = dims.c()
    _lib.check(_lib.load().rssm_ring_sizes(ctypes.byref(d), int(gdn), out), "rssm_ring_sizes")
    return list(out)


def rssm_ring_pointers(dims: Dims, ring: Ring, head=None, count=None, pending=None, rows_view=False,
                       stream=None):
    """Write the ring pointers of the call's batch entries (int32 [B] each, any
    may be None) on the device; ``rows_view`` reads pool rows 0..B-1 directly,
    ignoring the ring's slot map."""
    d = dims.c()
    if rows_view:
        if dims.batch != ring.rows:
            raise ValueError("rows_view needs batch == ring.rows")
        rc = ring.c()
        rc.slots = None
    else:
        rc = _ring_args(dims, ring, ring.gdn)
    outs = [_p(t, name, _I32, (dims.batch,), allow_none=True)
            for t, name in ((head, "head"), (count, "count"), (pending, "pending"))]
    _lib.check(_lib.load().rssm_ring_pointers(ctypes.byref(d), ctypes.byref(rc), *outs, _stream(stream)),
               "rssm_ring_pointers")


def rssm_ring_reset(dims: Dims, ring: Ring, mask=None, stream=None):
    d, rc = dims.c(), _ring_args(dims, ring, ring.gdn)
    m = _p(mask, "mask", _I32, (dims.batch,), allow_none=True)
    _lib.check(_lib.load().rssm_ring_reset(ctypes.byref(d), ctypes.byref(rc), m, _stream(stream)),
               "rssm_ring_reset")


# ------------------------------------------------------------------ Mamba-2
def ssm_decode_step(dims: Dims, state, v, k, q, dt, dt_bias, A, y, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d = dims.c()
    args = (_p(state, "state", _F32, (B, H, D, N)), _p(v, "v", _BF16, (B, H, D)),
            _p(k, "k", _BF16, (B, G, N)), _p(q, "q", _BF16, (B, G, N)),
            _p(dt, "dt", _F32, (B, H)), _p(dt_bias, "dt_bias", _F32, (H,)),
            _p(A, "A", _F32, (H,)), _p(y, "y", _F32, (B, H, D)))
    _lib.check(_lib.load().ssm_decode_step(ctypes.byref(d), *args, _stream(stream)), "ssm_decode_step")


def _ring_args(dims: Dims, ring: Ring, gdn: bool):
    if ring.gdn != gdn:
        raise ValueError("ring kind does not match the call (Mamba-2 vs GDN)")
    if dataclasses.replace(ring.dims, batch=dims.batch) != dims:
        raise ValueError("ring was allocated for different dims")
    if ring.slots is None and dims.batch != ring.rows:
        raise ValueError("batch differs from the ring's rows and no slot map is set")
    if ring.slots is not None and tuple(ring.slots.shape) != (dims.batch,):
        raise ValueError("slot map length differs from the batch")
    return ring.c()


def replay_append_decode(dims: Dims, state0, ring: Ring, v, k, q, dt, dt_bias, A, y,
                         flushed=None, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, False)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(v, "v", _BF16, (B, H, D)), _p(k, "k", _BF16, (B, G, N)),
            _p(q, "q", _BF16, (B, G, N)), _p(dt, "dt", _F32, (B, H)),
            _p(dt_bias, "dt_bias", _F32, (H,)), _p(A, "A", _F32, (H,)),
            _p(y, "y", dims.y_dtypes, (B, H, D)), _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().replay_append_decode(ctypes.byref(d), *args, _stream(stream)),
               "replay_append_decode")


def replay_append_decode_conv(dims: Dims, state0, ring: Ring, conv_state_in, conv_state_out, xbc, conv_w,
                              dt, dt_bias, A, y, flushed=None, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    C = H * D + 2 * G * N
    d, rc = dims.c(), _ring_args(dims, ring, False)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(conv_state_in, "conv_state_in", _BF16, (ring.rows, C, 3)),
            _p(conv_state_out, "conv_state_out", _BF16, (ring.rows, C, 3)),
            _p(xbc, "xbc", _BF16, (B, C)), _p(conv_w, "conv_w", _BF16, (C, 4)),
            _p(dt, "dt", _F32, (B, H)), _p(dt_bias, "dt_bias", _F32, (H,)), _p(A, "A", _F32, (H,)),
            _p(y, "y", dims.y_dtypes, (B, H, D)), _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().replay_append_decode_conv(ctypes.byref(d), *args, _stream(stream)),
               "replay_append_decode_conv")


def replay_flush(dims: Dims, state0, ring: Ring, mask=None, stream=None):
    B, H, D, N = dims.batch, dims.nheads, dims.head_dim, dims.state_dim
    d, rc = dims.c(), _ring_args(dims, ring, False)
    _lib.check(_lib.load().replay_flush(
        ctypes.byref(d), _p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
        _p(mask, "mask", _I32, (B,), allow_none=True), _stream(stream)), "replay_flush")


def replay_verify_T(dims: Dims, T: int, state0, ring: Ring, v, k, q, dt, dt_bias, A, y,
                    flushed=None, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, False)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(v, "v", _BF16, (B, T, H, D)), _p(k, "k", _BF16, (B, T, G, N)),
            _p(q, "q", _BF16, (B, T, G, N)), _p(dt, "dt", _F32, (B, T, H)),
            _p(dt_bias, "dt_bias", _F32, (H,)), _p(A, "A", _F32, (H,)),
            _p(y, "y", dims.y_dtypes, (B, T, H, D)), _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().replay_verify_T(ctypes.byref(d), int(T), *args, _stream(stream)),
               "replay_verify_T")


def replay_commit_verify_T(dims: Dims, T: int, state0, ring: Ring, accepted, v, k, q, dt, dt_bias, A, y,
                           flushed=None, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, False)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(accepted, "accepted", _I32, (B,)),
            _p(v, "v", _BF16, (B, T, H, D)), _p(k, "k", _BF16, (B, T, G, N)),
            _p(q, "q", _BF16, (B, T, G, N)), _p(dt, "dt", _F32, (B, T, H)),
            _p(dt_bias, "dt_bias", _F32, (H,)), _p(A, "A", _F32, (H,)),
            _p(y, "y", dims.y_dtypes, (B, T, H, D)), _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().replay_commit_verify_T(ctypes.byref(d), int(T), *args, _stream(stream)),
               "replay_commit_verify_T")


def replay_rollback(dims: Dims, ring: Ring, accepted, stream=None):
    d, rc = dims.c(), _ring_args(dims, ring, ring.gdn)
    _lib.check(_lib.load().replay_rollback(
        ctypes.byref(d), ctypes.byref(rc), _p(accepted, "accepted", _I32, (dims.batch,)),
        _stream(stream)), "replay_rollback")


# ------------------------------------------------------------------ Gated DeltaNet
def gdn_decode_step(dims: Dims, state, v, k, q, g, beta, y, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d = dims.c()
    args = (_p(state, "state", _F32, (B, H, D, N)), _p(v, "v", _BF16, (B, H, D)),
            _p(k, "k", _BF16, (B, G, N)), _p(q, "q", _BF16, (B, G, N)),
            _p(g, "g", _F32, (B, H)), _p(beta, "beta", _F32, (B, H)), _p(y, "y", _F32, (B, H, D)))
    _lib.check(_lib.load().gdn_decode_step(ctypes.byref(d), *args, _stream(stream)), "gdn_decode_step")


def gdn_replay_verify_T(dims: Dims, T: int, state0, ring: Ring, v, k, q, g, beta, y,
                        flushed=None, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, True)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(v, "v", _BF16, (B, T, H, D)), _p(k, "k", _BF16, (B, T, G, N)),
            _p(q, "q", _BF16, (B, T, G, N)), _p(g, "g", _F32, (B, T, H)),
            _p(beta, "beta", _F32, (B, T, H)), _p(y, "y", dims.y_dtypes, (B, T, H, D)),
            _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().gdn_replay_verify_T(ctypes.byref(d), int(T), *args, _stream(stream)),
               "gdn_replay_verify_T")


def gdn_replay_commit_verify_T(dims: Dims, T: int, state0, ring: Ring, accepted, v, k, q, g, beta, y,
                               flushed=None, stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, True)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(accepted, "accepted", _I32, (B,)),
            _p(v, "v", _BF16, (B, T, H, D)), _p(k, "k", _BF16, (B, T, G, N)),
            _p(q, "q", _BF16, (B, T, G, N)), _p(g, "g", _F32, (B, T, H)),
            _p(beta, "beta", _F32, (B, T, H)), _p(y, "y", dims.y_dtypes, (B, T, H, D)),
            _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().gdn_replay_commit_verify_T(ctypes.byref(d), int(T), *args, _stream(stream)),
               "gdn_replay_commit_verify_T")


def gdn_replay_append_decode(dims: Dims, state0, ring: Ring, v, k, q, g, beta, y, flushed=None,
                             stream=None):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, True)
    args = (_p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(v, "v", _BF16, (B, H, D)), _p(k, "k", _BF16, (B, G, N)), _p(q, "q", _BF16, (B, G, N)),
            _p(g, "g", _F32, (B, H)), _p(beta, "beta", _F32, (B, H)), _p(y, "y", dims.y_dtypes, (B, H, D)),
            _p(flushed, "flushed", _I32, (B,), allow_none=True))
    _lib.check(_lib.load().gdn_replay_append_decode(ctypes.byref(d), *args, _stream(stream)),
               "gdn_replay_append_decode")


def gdn_replay_flush(dims: Dims, state0, ring: Ring, mask=None, stream=None):
    B, H, D, N = dims.batch, dims.nheads, dims.head_dim, dims.state_dim
    d, rc = dims.c(), _ring_args(dims, ring, True)
    _lib.check(_lib.load().gdn_replay_flush(
        ctypes.byref(d), _p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
        _p(mask, "mask", _I32, (B,), allow_none=True), _stream(stream)), "gdn_replay_flush")


# ------------------------------------------------------------------ snapshot baseline
def _snapshot_args(dims: Dims, T: int, pool, slot, v, k, q, err):
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    if not isinstance(pool, torch.Tensor) or pool.dim() != 5:
        raise ValueError("pool must be a [B, P, H, d, n] tensor")
    P = int(pool.shape[1])
    return P, (_p(pool, "pool", _F32, (B, P, H, D, N)), _p(slot, "slot", _I32, (B,)),
               _p(v, "v", _BF16, (B, T, H, D)), _p(k, "k", _BF16, (B, T, G, N)),
               _p(q, "q", _BF16, (B, T, G, N)))


def ssm_snapshot_verify_T(dims: Dims, T: int, pool, slot, v, k, q, dt, dt_bias, A, y, err=None,
                          stream=None):
    B, H, D = dims.batch, dims.nheads, dims.head_dim
    P, args = _snapshot_args(dims, T, pool, slot, v, k, q, err)
    rest = (_p(dt, "dt", _F32, (B, T, H)), _p(dt_bias, "dt_bias", _F32, (H,)), _p(A, "A", _F32, (H,)),
            _p(y, "y", _F32, (B, T, H, D)), _p(err, "err", _I32, (1,), allow_none=True))
    _lib.check(_lib.load().ssm_snapshot_verify_T(ctypes.byref(dims.c()), int(T), P, *args, *rest,
                                                 _stream(stream)), "ssm_snapshot_verify_T")


def gdn_snapshot_verify_T(dims: Dims, T: int, pool, slot, v, k, q, g, beta, y, err=None, stream=None):
    B, H, D = dims.batch, dims.nheads, dims.head_dim
    P, args = _snapshot_args(dims, T, pool, slot, v, k, q, err)
    rest = (_p(g, "g", _F32, (B, T, H)), _p(beta, "beta", _F32, (B, T, H)),
            _p(y, "y", _F32, (B, T, H, D)), _p(err, "err", _I32, (1,), allow_none=True))
    _lib.check(_lib.load().gdn_snapshot_verify_T(ctypes.byref(dims.c()), int(T), P, *args, *rest,
                                                 _stream(stream)), "gdn_snapshot_verify_T")


def snapshot_commit(T: int, nslots: int, slot, accepted, err=None, stream=None):
    B = int(slot.shape[0])
    _lib.check(_lib.load().snapshot_commit(
        B, int(T), int(nslots), _p(slot, "slot", _I32, (B,)), _p(accepted, "accepted", _I32, (B,)),
        _p(err, "err", _I32, (1,), allow_none=True), _stream(stream)), "snapshot_commit")


# ------------------------------------------------------------------ conv1d
def causal_conv1d_update(conv_state, x, weight, out, stream=None):
    if conv_state.dim() != 3:
        raise ValueError("conv_state must be [B, C, W-1]")
    B, C, Wm1 = conv_state.shape
    W = Wm1 + 1
    args = (_p(conv_state, "conv_state", _BF16, (B, C, Wm1)), _p(x, "x", _BF16, (B, C)),
            _p(weight, "weight", _BF16, (C, W)), _p(out, "out", _F32, (B, C)))
    _lib.check(_lib.load().causal_conv1d_update(B, C, W, *args, _stream(stream)),
               "causal_conv1d_update")


# ------------------------------------------------------------------ probes
def rssm_probe_copy(dst, src, stream=None):
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _lib.check(_lib.load().rssm_probe_copy(dst.data_ptr(), src.data_ptr(), n, _stream(stream)),
               "rssm_probe_copy")


def rssm_probe_read(src, sink, stream=None):
    n = src.numel() * src.element_size()
    need = _lib.load().rssm_probe_read_sink_floats(n)
    if sink.dtype != torch.float32 or sink.numel() < need:
        raise ValueError(f"sink must be fp32 with >= {need} elements")
    _lib.check(_lib.load().rssm_probe_read(src.data_ptr(), n, sink.data_ptr(), _stream(stream)),
               "rssm_probe_read")


def probe_read_sink_floats(nbytes: int) -> int:
    return int(_lib.load().rssm_probe_read_sink_floats(nbytes))


# ------------------------------------------------------------------ prepared calls
class Prepared:
    """A library call with every pointer argument resolved once.

    Calling it re-issues the same C call (same buffers, same stream) with no
    per-call marshalling, for tight timing loops and graph capture."""

    def __init__(self, fn, *args, keep=()):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _lib.check(rc, self._fn.__name__)


def prepare_replay_append_decode(dims: Dims, state0, ring: Ring, v, k, q, dt, dt_bias, A, y,
                                 flushed=None, stream=None) -> Prepared:
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d, rc = dims.c(), _ring_args(dims, ring, False)
    args = (ctypes.byref(d), _p(state0, "state0", _F32, (ring.rows, H, D, N)), ctypes.byref(rc),
            _p(v, "v", _BF16, (B, H, D)), _p(k, "k", _BF16, (B, G, N)),
            _p(q, "q", _BF16, (B, G, N)), _p(dt, "dt", _F32, (B, H)),
            _p(dt_bias, "dt_bias", _F32, (H,)), _p(A, "A", _F32, (H,)),
            _p(y, "y", dims.y_dtypes, (B, H, D)), _p(flushed, "flushed", _I32, (B,), allow_none=True),
            _stream(stream))
    return Prepared(_lib.load().replay_append_decode, *args, keep=(d, rc))


def prepare_ssm_decode_step(dims: Dims, state, v, k, q, dt, dt_bias, A, y, stream=None) -> Prepared:
    B, H, D, N, G = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups
    d = dims.c()
    args = (ctypes.byref(d), _p(state, "state", _F32, (B, H, D, N)), _p(v, "v", _BF16, (B, H, D)),
            _p(k, "k", _BF16, (B, G, N)), _p(q, "q", _BF16, (B, G, N)),
            _p(dt, "dt", _F32, (B, H)), _p(dt_bias, "dt_bias", _F32, (H,)),
            _p(A, "A", _F32, (H,)), _p(y, "y", _F32, (B, H, D)), _stream(stream))
    return Prepared(_lib.load().ssm_decode_step, *args, keep=(d,))


def prepare_causal_conv1d_update(conv_state, x, weight, out, stream=None) -> Prepared:
    B, C, Wm1 = conv_state.shape
    args = (B, C, Wm1 + 1, _p(conv_state, "conv_state", _BF16, (B, C, Wm1)),
            _p(x, "x", _BF16, (B, C)), _p(weight, "weight", _BF16, (C, Wm1 + 1)),
            _p(out, "out", _F32, (B, C)), _stream(stream))
    return Prepared(_lib.load().causal_conv1d_update, *args)
