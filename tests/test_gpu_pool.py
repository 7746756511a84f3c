"""Pooled rings through the C ABI: the checkpoints, rings and records live in a
pool of request rows, and each call maps its batch entries to rows with a slot
map that changes from call to call (requests reordered, padding entries).

Each request is followed by its own oracle run on the inputs of whatever batch
position it held at each call.  Checked: y of live entries (1e-3), the
checkpoint at every flush and after a final flush (1e-4), the pointers of every
used row (bit-exact), padding entries' outputs untouched, and rows no call
names left bit-identical."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4
ROWS = 7
# slot maps per call (batch of 4): requests live in rows 5, 0 and 3; -1 = padding
MAPS = [[5, 0, 3, -1], [3, -1, 5, 0], [0, 3, -1, 5], [-1, 5, 0, 3]]
USED = (0, 3, 5)


def _dims(sh):
    return rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity)


def _pool_state(sh, seed, cfg):
    return synth.state0(sh.with_(batch=ROWS), seed, cfg)


def _sub(st, b, spec):
    """Batch position b of a step's (or round's) float64 inputs, as a batch of one."""
    return {k: v[b:b + 1] for k, v in st.items()}


@pytest.mark.parametrize("L", [4, 16])
def test_pooled_append_decode(L):
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(capacity=L)               # B = 4 positions, H = 8, d = 64, G = 1
    seed, steps = base.cfg_seed, 3 * L + 2
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = _pool_state(sh, seed, 0)
    dims = _dims(sh)
    ring = rd.Ring(dims, rows=ROWS)
    state0 = dev_f32(S0)
    untouched = state0.clone()
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = {r: S0[r:r + 1].astype(np.float64) for r in USED}
    count = {r: 0 for r in USED}
    for t in range(steps):
        mp = MAPS[t % len(MAPS)]
        ring.use_slots(dev_i32(np.array(mp)))
        st = synth.mamba2_step_inputs(sh, seed, 0, t)
        y.fill_(float("nan"))
        flushed.fill_(7)
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                                dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y, flushed)
        s64 = mamba2_step_f64(st)
        yh, fh = y.cpu().numpy(), flushed.cpu().numpy()
        for b, r in enumerate(mp):
            if r < 0:
                assert np.isnan(yh[b]).all() and fh[b] == 7, (t, b)
                continue
            sb = _sub(s64, b, False)
            delta, a = o_m2.step_size_and_decay(sb["dt"], dt_bias.astype(np.float64), A.astype(np.float64))
            S[r], y_ref = o_m2.standard_step(S[r], sb["v"], sb["k"], sb["q"], delta, a, sh.ngroups)
            assert rel_err(yh[b], y_ref[0]) <= Y_TOL, (t, b)
            count[r] += 1
            fl = count[r] == L
            assert fh[b] == int(fl), (t, b)
            if fl:
                count[r] = 0
                assert rel_err(state0[r].cpu().numpy(), S[r][0]) <= S_TOL, (t, r)
        ring.use_slots(None)
        cnt = ring.count.cpu().numpy()
        for r in USED:
            assert cnt[r] == count[r], (t, r)
    assert int(ring.err.item()) == 0
    for r in set(range(ROWS)) - set(USED):
        assert torch.equal(state0[r], untouched[r])
        assert torch.all(ring.meta[r] == 0)
    # explicit flush and reset through the slot map (padding skipped)
    ring.use_slots(dev_i32(np.array(MAPS[0])))
    rd.replay_flush(dims, state0, ring)
    for r in USED:
        assert rel_err(state0[r].cpu().numpy(), S[r][0]) <= S_TOL
    rd.rssm_ring_reset(dims, ring)
    ring.use_slots(None)
    assert torch.all(ring.count == 0) and int(ring.err.item()) == 0


def test_pooled_verify_rollback():
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=4, nheads=8, capacity=16, T=4)
    seed, R, T, L = base.cfg_seed, 20, 4, 16
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = _pool_state(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims, rows=ROWS)
    state0 = dev_f32(S0)
    untouched = state0.clone()
    y = torch.empty(sh.batch, T, sh.nheads, sh.head_dim, device="cuda")
    S = {r: S0[r:r + 1].astype(np.float64) for r in USED}
    for rnd in range(R):
        mp = MAPS[rnd % len(MAPS)]
        ring.use_slots(dev_i32(np.array(mp)))
        st = synth.mamba2_step_inputs(sh, seed, 2, rnd)
        y.fill_(float("nan"))
        rd.replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                           dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        rd.replay_rollback(dims, ring, dev_i32(acc[rnd]))
        s64 = mamba2_step_f64(st)
        yh = y.cpu().numpy()
        for b, r in enumerate(mp):
            if r < 0:
                assert np.isnan(yh[b]).all()
                continue
            y_ref, S[r] = o_m2.spec_round_snapshot(S[r], _sub(s64, b, True), dt_bias.astype(np.float64),
                                                   A.astype(np.float64), sh.ngroups, acc[rnd, b:b + 1])
            assert rel_err(yh[b], y_ref[0]) <= Y_TOL, (rnd, b)
    ring.use_slots(dev_i32(np.array(MAPS[0])))
    rd.replay_flush(dims, state0, ring)
    ring.use_slots(None)
    assert int(ring.err.item()) == 0
    for r in USED:
        assert rel_err(state0[r].cpu().numpy(), S[r][0]) <= S_TOL
    for r in set(range(ROWS)) - set(USED):
        assert torch.equal(state0[r], untouched[r])


@pytest.mark.parametrize("mode", ["verify", "append"])
def test_pooled_gdn(mode):
    base = synth.WORKLOADS[4]
    T = 2 if mode == "verify" else 1
    sh = base.shape.with_(batch=4, nheads=8, ngroups=8, capacity=8, T=T)
    seed, R, L = base.cfg_seed, 14, 8
    S0 = _pool_state(sh, seed, 4)
    acc = synth.accept_draws(seed, 4, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims, gdn=True, rows=ROWS)
    state0 = dev_f32(S0)
    untouched = state0.clone()
    S = {r: S0[r:r + 1].astype(np.float64) for r in USED}
    for rnd in range(R):
        mp = MAPS[rnd % len(MAPS)]
        ring.use_slots(dev_i32(np.array(mp)))
        st = synth.gdn_round_inputs(sh, seed, 4, rnd)
        if mode == "verify":
            y = torch.full((sh.batch, T, sh.nheads, sh.head_dim), float("nan"), device="cuda")
            rd.gdn_replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                                   dev_f32(st["g"]), dev_f32(st["beta"]), y)
            rd.replay_rollback(dims, ring, dev_i32(acc[rnd]))
        else:
            st = {k_: np.ascontiguousarray(v_[:, 0]) for k_, v_ in st.items()}
            y = torch.full((sh.batch, sh.nheads, sh.head_dim), float("nan"), device="cuda")
            rd.gdn_replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                        dev_bf16(st["q"]), dev_f32(st["g"]), dev_f32(st["beta"]), y)
        s64 = gdn_step_f64(st)
        yh = y.cpu().numpy()
        for b, r in enumerate(mp):
            if r < 0:
                assert np.isnan(yh[b]).all()
                continue
            sb = _sub(s64, b, True)
            if mode == "verify":
                y_ref, S[r] = o_gdn.spec_round_snapshot(S[r], sb, sh.ngroups, acc[rnd, b:b + 1])
            else:
                S[r], y_ref = o_gdn.householder_step(S[r], sb["v"], sb["k"], sb["q"], sb["g"], sb["beta"],
                                                     sh.ngroups)
            assert rel_err(yh[b], y_ref[0]) <= Y_TOL, (rnd, b)
    ring.use_slots(dev_i32(np.array(MAPS[0])))
    rd.gdn_replay_flush(dims, state0, ring)
    ring.use_slots(None)
    assert int(ring.err.item()) == 0
    for r in USED:
        assert rel_err(state0[r].cpu().numpy(), S[r][0]) <= S_TOL
    for r in set(range(ROWS)) - set(USED):
        assert torch.equal(state0[r], untouched[r])


def test_slot_outside_pool_is_skipped_and_flagged():
    base = synth.WORKLOADS[0]
    sh = base.shape
    A, dt_bias = synth.mamba2_head_params(sh, base.cfg_seed, 0)
    dims = _dims(sh)
    ring = rd.Ring(dims, rows=ROWS)
    state0 = dev_f32(_pool_state(sh, base.cfg_seed, 0))
    before = state0.clone()
    ring.use_slots(dev_i32(np.array([ROWS, 2, ROWS + 5, -3])))
    st = synth.mamba2_step_inputs(sh, base.cfg_seed, 0, 0)
    y = torch.full((sh.batch, sh.nheads, sh.head_dim), float("nan"), device="cuda")
    rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                            dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
    rd.replay_rollback(dims, ring, dev_i32(np.zeros(sh.batch, int)))
    torch.cuda.synchronize()
    assert int(ring.err.item()) == 8                   # RSSM_ERR_SLOT
    yh = y.cpu().numpy()
    assert np.isnan(yh[[0, 2, 3]]).all() and np.isfinite(yh[1]).all()
    ring.use_slots(None)
    assert ring.count.cpu().tolist() == [0, 0, 1, 0, 0, 0, 0]
    assert torch.equal(state0, before)


def test_pooled_commit_verify():
    """One launch per round on pooled rows whose batch positions change every call:
    accepted[b] carries the previous window of the request now at position b."""
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=4, nheads=8, capacity=16, T=4)
    seed, R, T = base.cfg_seed, 18, 4
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = _pool_state(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims, rows=ROWS)
    state0 = dev_f32(S0)
    untouched = state0.clone()
    y = torch.empty(sh.batch, T, sh.nheads, sh.head_dim, device="cuda")
    S = {r: S0[r:r + 1].astype(np.float64) for r in USED}
    last = {r: 0 for r in USED}                   # each row's window awaiting its commit
    for rnd in range(R):
        mp = MAPS[rnd % len(MAPS)]
        ring.use_slots(dev_i32(np.array(mp)))
        prev = np.array([last[r] if r >= 0 else 0 for r in mp], dtype=np.int32)
        st = synth.mamba2_step_inputs(sh, seed, 2, rnd)
        y.fill_(float("nan"))
        rd.replay_commit_verify_T(dims, T, state0, ring, dev_i32(prev), dev_bf16(st["v"]), dev_bf16(st["k"]),
                                  dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        s64 = mamba2_step_f64(st)
        yh = y.cpu().numpy()
        for b, r in enumerate(mp):
            if r < 0:
                assert np.isnan(yh[b]).all()
                continue
            y_ref, S[r] = o_m2.spec_round_snapshot(S[r], _sub(s64, b, True), dt_bias.astype(np.float64),
                                                   A.astype(np.float64), sh.ngroups, acc[rnd, b:b + 1])
            assert rel_err(yh[b], y_ref[0]) <= Y_TOL, (rnd, b)
            last[r] = int(acc[rnd, b])
    mp = MAPS[0]
    ring.use_slots(dev_i32(np.array(mp)))
    rd.replay_rollback(dims, ring, dev_i32(np.array([last[r] if r >= 0 else 0 for r in mp], dtype=np.int32)))
    rd.replay_flush(dims, state0, ring)
    ring.use_slots(None)
    assert int(ring.err.item()) == 0
    for r in USED:
        assert rel_err(state0[r].cpu().numpy(), S[r][0]) <= S_TOL
    for r in set(range(ROWS)) - set(USED):
        assert torch.equal(state0[r], untouched[r])


def test_pooled_fused_front_end():
    """The fused front-end on pooled rows: the conv states live in the pool's rows
    (ping-pong buffers), the tokens at the batch positions of each call."""
    from oracle import conv1d as o_conv
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(batch=4, nheads=8, ngroups=2, capacity=8)
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    C = H * D + 2 * G * N
    seed, steps = base.cfg_seed, 2 * L + 3
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = _pool_state(sh, seed, 0)
    cs_bits, w_bits = synth.conv_layer(ROWS, C, 4, seed, 0)
    dims = _dims(sh)
    ring = rd.Ring(dims, rows=ROWS)
    state0 = dev_f32(S0)
    untouched = state0.clone()
    cs = [dev_bf16(cs_bits), dev_bf16(cs_bits)]
    w = dev_bf16(w_bits)
    y = torch.empty(B, H, D, device="cuda")
    S = {r: S0[r:r + 1].astype(np.float64) for r in USED}
    cs64 = {r: synth.bf16_bits_to_f64(cs_bits[r:r + 1]) for r in USED}
    W64 = synth.bf16_bits_to_f64(w_bits)
    for t in range(steps):
        mp = MAPS[t % len(MAPS)]
        ring.use_slots(dev_i32(np.array(mp)))
        x_bits = synth.conv_step_input(B, C, seed, 0, t)
        dt = synth.mamba2_step_inputs(sh, seed, 0, t)["dt"]
        cin, cout = cs[t % 2], cs[(t + 1) % 2]
        y.fill_(float("nan"))
        rd.replay_append_decode_conv(dims, state0, ring, cin, cout, dev_bf16(x_bits), w, dev_f32(dt),
                                     dev_f32(dt_bias), dev_f32(A), y)
        yh = y.cpu().numpy()
        got = cout.view(torch.int16).cpu().numpy().view(np.uint16)
        x64 = synth.bf16_bits_to_f64(x_bits)
        for b, r in enumerate(mp):
            if r < 0:
                assert np.isnan(yh[b]).all()
                continue
            out, cs64[r] = o_conv.update(cs64[r], x64[b:b + 1], W64)
            v, k, q = o_conv.split_xbc(o_conv.round_bf16(out), H, D, G, N)
            delta, a = o_m2.step_size_and_decay(dt[b:b + 1].astype(np.float64), dt_bias.astype(np.float64),
                                                A.astype(np.float64))
            S[r], y_ref = o_m2.standard_step(S[r], v, k, q, delta, a, G)
            assert rel_err(yh[b], y_ref[0]) <= Y_TOL, (t, b)
            assert np.array_equal(synth.bf16_bits_to_f64(got[r:r + 1]), cs64[r]), (t, r)
    ring.use_slots(None)
    assert int(ring.err.item()) == 0
    for r in set(range(ROWS)) - set(USED):
        assert torch.equal(state0[r], untouched[r])
