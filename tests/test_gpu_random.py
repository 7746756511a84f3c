"""Seeded random configurations through the C ABI, against the oracle.

Each case draws its own combination of what the other GPU tests exercise one at
a time: head dim, state size (Mamba-2), groups and heads per group, ring capacity, decode mode
(append-decode, or verify rounds with random acceptance and device-side
rollback), a pooled ring whose slot map changes every call (padding entries
included), explicit flushes of a random subset of requests between calls, and
the storage-precision flags.  Every request (pool row) is followed by its own
oracle object on the inputs of whatever batch position it held at each call.

Checked at every call: y of live entries; padding entries' outputs untouched;
the flush flags; head, count and pending of every row (bit-exact; rows no call
named stay zero); the checkpoint of every row that folded; at the end, every
row after a final flush.  Bars as elsewhere: y 1e-3 and fp32 state 1e-4, plus
the derived bf16 terms where a flag asks for bf16 storage (2^-8 for bf16 y;
1e-3 + 2^-7 for y and states once GDN corrections are cached in bf16)."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from oracle import replay as o_rep
from ssm_recurrent_decode_amd import _lib, synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

NCASES = 16


def _case(i):
    rng = np.random.default_rng(90_000 + i)
    gdn = i % 2 == 1
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4]))
    hpg = int(rng.choice([1, 2])) if gdn else int(rng.choice([1, 2, 4]))
    L = int(rng.integers(2, 33))
    verify = bool(rng.random() < 0.6)
    T = int(rng.integers(1, min(8, L // 2) + 1)) if verify else 1
    B = int(rng.integers(1, 5 if gdn else 6))
    pooled = bool(rng.random() < 0.5)
    rows = B + int(rng.integers(0, 3)) if pooled else B
    flags = 0
    if rng.random() < 0.3:
        flags |= _lib.RSSM_F_Y_BF16
    if gdn and rng.random() < 0.3:
        flags |= _lib.RSSM_F_U_BF16
    seed = int(rng.integers(1 << 30))
    n = 128 if gdn else (128, 64, 128, 256)[(i // 2) % 4]   # GDN is built for n = 128
    return dict(gdn=gdn, d=d, n=n, G=G, H=G * hpg, L=L, verify=verify, T=T, B=B, pooled=pooled, rows=rows,
                flags=flags, seed=seed)


def _slot_map(rng, B, rows, pooled):
    if not pooled:
        return None
    mp = rng.permutation(rows)[:B].astype(np.int32)
    if B > 1 and rng.random() < 0.3:
        mp[int(rng.integers(B))] = -1           # a padding entry
    return mp


@pytest.mark.parametrize("i", range(NCASES))
def test_random_configuration(i):
    cf = _case(i)
    gdn, d, G, H, L, T, B, rows = cf["gdn"], cf["d"], cf["G"], cf["H"], cf["L"], cf["T"], cf["B"], cf["rows"]
    verify, flags, seed = cf["verify"], cf["flags"], cf["seed"]
    ybf, ubf = bool(flags & _lib.RSSM_F_Y_BF16), bool(flags & _lib.RSSM_F_U_BF16)
    cid = 4 if gdn else 2
    sh = synth.WORKLOADS[cid].shape.with_(batch=B, nheads=H, head_dim=d, state_dim=cf["n"], ngroups=G, capacity=L,
                                          T=T)
    y_tol = (1e-3 + 2.0**-7 if ubf else 1e-3) + (2.0**-8 if ybf else 0.0)
    s_tol = 1e-3 + 2.0**-7 if ubf else 1e-4
    rng = np.random.default_rng(seed)

    S0 = synth.state0(sh.with_(batch=rows), seed, cid)
    dims = rd.Dims(B, H, d, sh.state_dim, G, L, flags=flags)
    ring = rd.Ring(dims, gdn=gdn, rows=rows if cf["pooled"] else None)
    state0 = dev_f32(S0)
    if gdn:
        reqs = [o_gdn.GDNReplayRequest(S0[r].astype(np.float64), L, G, u_bf16=ubf) for r in range(rows)]
    else:
        A, dt_bias = synth.mamba2_head_params(sh, seed, cid)
        A64, bias64 = A.astype(np.float64), dt_bias.astype(np.float64)
        Ad, biasd = dev_f32(A), dev_f32(dt_bias)
        reqs = [o_rep.ReplayRequest(S0[r].astype(np.float64), L, G) for r in range(rows)]
    ydt = torch.bfloat16 if ybf else torch.float32
    y = torch.empty((B, T, H, d) if verify else (B, H, d), dtype=ydt, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    calls = 12 if verify else 2 * L + 2
    acc = synth.accept_draws(seed, cid, calls, B, T)

    def check_rows(tag):
        h, c, p = ring.head.cpu().numpy(), ring.count.cpu().numpy(), ring.pending.cpu().numpy()
        for r in range(rows):
            assert (h[r], c[r], p[r]) == (reqs[r].head, reqs[r].count, reqs[r].pending), (tag, r)
        assert ring.copies_agree(), tag

    def check_state(r, tag):
        e = rel_err(state0[r].cpu().numpy(), reqs[r].S0)
        assert e <= s_tol, (tag, r, e)

    for t in range(calls):
        mp = _slot_map(rng, B, rows, cf["pooled"])
        ring.use_slots(None if mp is None else dev_i32(mp))
        rows_of = list(range(B)) if mp is None else [int(x) for x in mp]

        # an explicit flush of a random subset of the requests, every fifth call
        if t % 5 == 4:
            mask = (rng.random(B) < 0.5).astype(np.int32)
            if gdn:
                rd.gdn_replay_flush(dims, state0, ring, dev_i32(mask))
            else:
                rd.replay_flush(dims, state0, ring, dev_i32(mask))
            for b, r in enumerate(rows_of):
                if r >= 0 and mask[b] and reqs[r].flush():
                    check_state(r, ("explicit flush", t))
            check_rows(("explicit flush", t))

        if gdn:
            st = synth.gdn_round_inputs(sh, seed, cid, t)
            if not verify:
                st = {k_: np.ascontiguousarray(v_[:, 0]) for k_, v_ in st.items()}
            s64 = gdn_step_f64(st)
            dv = {k_: (dev_bf16(v_) if v_.dtype == np.uint16 else dev_f32(v_)) for k_, v_ in st.items()}
        else:
            st = synth.mamba2_step_inputs(sh, seed, cid, t)
            if verify and T == 1:
                st = {k_: v_[:, None] for k_, v_ in st.items()}
            s64 = mamba2_step_f64(st)
            dv = {k_: (dev_bf16(v_) if v_.dtype == np.uint16 else dev_f32(v_)) for k_, v_ in st.items()}
            delta, a = o_m2.step_size_and_decay(s64["dt"], bias64, A64)

        y.fill_(float("nan"))
        flushed.fill_(7)
        if gdn and verify:
            rd.gdn_replay_verify_T(dims, T, state0, ring, dv["v"], dv["k"], dv["q"], dv["g"], dv["beta"], y,
                                   flushed)
        elif gdn:
            rd.gdn_replay_append_decode(dims, state0, ring, dv["v"], dv["k"], dv["q"], dv["g"], dv["beta"], y,
                                        flushed)
        elif verify:
            rd.replay_verify_T(dims, T, state0, ring, dv["v"], dv["k"], dv["q"], dv["dt"], biasd, Ad, y, flushed)
        else:
            rd.replay_append_decode(dims, state0, ring, dv["v"], dv["k"], dv["q"], dv["dt"], biasd, Ad, y,
                                    flushed)
        yh, fh = y.float().cpu().numpy(), flushed.cpu().numpy()
        for b, r in enumerate(rows_of):
            if r < 0:
                assert np.isnan(yh[b]).all() and fh[b] == 7, (t, b)
                continue
            if gdn and verify:
                y_ref, _, fl = reqs[r].verify_round(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b],
                                                    s64["beta"][b])
            elif gdn:
                y_ref, fl = reqs[r].decode_step(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b],
                                                s64["beta"][b])
            elif verify:
                y_ref, fl = reqs[r].verify_round(s64["v"][b], s64["k"][b], s64["q"][b], delta[b], a[b])
            else:
                y_ref, fl = reqs[r].decode_step(s64["v"][b], s64["k"][b], s64["q"][b], delta[b], a[b])
            e = rel_err(yh[b], y_ref)
            assert e <= y_tol, (t, b, e)
            assert fh[b] == int(fl), (t, b)
            if fl:
                check_state(r, ("flush", t))
        if verify:
            rd.replay_rollback(dims, ring, dev_i32(acc[t]))
            for b, r in enumerate(rows_of):
                if r >= 0:
                    reqs[r].commit(int(acc[t, b]))
        check_rows(("call", t))
    assert int(ring.err.item()) == 0

    # every row after a final flush (batch = all rows, row = batch entry)
    ring.use_slots(None)
    all_dims = rd.Dims(rows, H, d, sh.state_dim, G, L, flags=flags)
    if gdn:
        rd.gdn_replay_flush(all_dims, state0, ring)
    else:
        rd.replay_flush(all_dims, state0, ring)
    for r in range(rows):
        reqs[r].flush()
        check_state(r, "final flush")
    check_rows("final flush")
    assert int(ring.err.item()) == 0
