"""GPU parity on small workloads, every entry point through the C ABI, against the
CPU oracle on the same seeded inputs.

Bars: y within max relative error 1e-3 and fp32 state within 1e-4 (error metric
in tests/util.rel_err); ring pointers, flush flags and committed counts bit-exact;
the conv state shift bit-exact."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import conv1d as o_conv
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from oracle import replay as o_rep
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4


def _dims(sh):
    return rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity)


def _mamba2_case(sh, seed, cfg_id, steps, ring_dominant=False):
    A, dt_bias = synth.mamba2_head_params(sh, seed, cfg_id)
    S0 = synth.state0(sh, seed, cfg_id)
    if ring_dominant:
        rng = np.random.default_rng(seed)
        A = -rng.uniform(0.1, 1.0, sh.nheads).astype(np.float32)
        dt_bias = np.zeros(sh.nheads, np.float32)
        S0 = np.zeros_like(S0)
    seq = [synth.mamba2_step_inputs(sh, seed, cfg_id, t) for t in range(steps)]
    return A, dt_bias, S0, seq


@pytest.mark.parametrize("d,G", [(64, 1), (128, 2)])
def test_ssm_decode_step_small(d, G):
    sh = synth.WORKLOADS[0].shape.with_(head_dim=d, ngroups=G)
    seed = synth.WORKLOADS[0].cfg_seed
    A, dt_bias, S0, seq = _mamba2_case(sh, seed, 0, 20)
    dims = _dims(sh)
    state = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    ys_ref, Ss_ref = o_m2.run_standard(S0.astype(np.float64), [mamba2_step_f64(s) for s in seq],
                                       dt_bias.astype(np.float64), A.astype(np.float64), G)
    for t, st in enumerate(seq):
        rd.ssm_decode_step(dims, state, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                           dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        assert rel_err(y.cpu().numpy(), ys_ref[t]) <= Y_TOL, t
    assert rel_err(state.cpu().numpy(), Ss_ref[-1]) <= S_TOL


@pytest.mark.parametrize("d,G,L,ring_dominant", [(64, 1, 8, False), (128, 2, 8, False),
                                                 (64, 2, 5, False), (64, 1, 8, True),
                                                 (128, 4, 32, True),
                                                 (64, 8, 1, False), (64, 1, 2, False)])  # every step / every other folds
def test_replay_append_decode_small(d, G, L, ring_dominant):
    """Config-0 workload (and variants): y every step, S_0 at every flush, pointers
    and flush flags every step, against the oracle."""
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(head_dim=d, ngroups=G, capacity=L)
    steps = max(base.steps, 2 * L + 3)
    A, dt_bias, S0, seq = _mamba2_case(sh, base.cfg_seed, 0, steps, ring_dominant)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    seq64 = [mamba2_step_f64(s) for s in seq]
    ys_ref, Ss_ref = o_m2.run_standard(S0.astype(np.float64), seq64, dt_bias.astype(np.float64),
                                       A.astype(np.float64), G)
    sched = o_rep.pointer_schedule_standard(L, steps)
    nflush = 0
    for t, st in enumerate(seq):
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A),
                                y, flushed)
        e = rel_err(y.cpu().numpy(), ys_ref[t])
        assert e <= Y_TOL, (t, e)
        head, count, fl = sched[t]
        assert torch.all(ring.head == head) and torch.all(ring.count == count), t
        assert torch.all(ring.pending == 0) and ring.copies_agree()
        assert torch.all(flushed == int(fl)), t
        if fl:
            nflush += 1
            es = rel_err(state0.cpu().numpy(), Ss_ref[t])
            assert es <= S_TOL, (t, es)
    assert nflush == steps // L
    assert int(ring.err.item()) == 0
    # explicit flush of whatever is cached equals the standard state
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), Ss_ref[-1]) <= S_TOL
    assert torch.all(ring.count == 0)


def test_ring_record_contents():
    """The per-head ring record after a few appends: every head's pointer word
    equal, word 2 the head's A, word 3 + slot the step size of the entry cached in
    that slot (against the oracle's softplus, at fp32 rounding); and the values
    cached in each slot, bit-exact."""
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(capacity=8)
    A, dt_bias, S0, seq = _mamba2_case(sh, base.cfg_seed, 0, 13, False)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    for st in seq:                       # 13 appends at L = 8: one flush, 5 cached
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
    torch.cuda.synchronize()
    meta = ring.meta.cpu().numpy()
    assert ring.copies_agree()
    head, count = int(ring.head[0].item()), int(ring.count[0].item())
    assert (head, count) == (0, 5)
    assert np.array_equal(meta[:, :, 2], np.broadcast_to(A.astype(np.float32), meta[:, :, 2].shape))
    for j in range(count):               # logical entry j is the append of step 8 + j
        delta, _ = o_m2.step_size_and_decay(seq[8 + j]["dt"], dt_bias, A)
        got = meta[:, :, 3 + (head + j) % sh.capacity].astype(np.float64)
        assert np.max(np.abs(got - delta) / np.abs(delta)) <= 2e-6, j
    # the cached values, bit for bit, through the head-blocked layout
    vals = ring.entries().view(torch.int16).cpu().numpy().view(np.uint16)
    for j in range(count):
        assert np.array_equal(vals[:, :, (head + j) % sh.capacity], seq[8 + j]["v"]), j
    assert int(ring.err.item()) == 0


def test_replay_append_decode_is_deterministic():
    base = synth.WORKLOADS[0]
    sh = base.shape
    A, dt_bias, S0, seq = _mamba2_case(sh, base.cfg_seed, 0, 12)
    dims = _dims(sh)
    outs = []
    for _ in range(2):
        ring = rd.Ring(dims)
        state0 = dev_f32(S0)
        y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
        ys = []
        for st in seq:
            rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                    dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias),
                                    dev_f32(A), y)
            ys.append(y.clone())
        outs.append((torch.stack(ys), state0.clone(), ring.vu.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2].view(torch.int16), outs[1][2].view(torch.int16))


def test_replay_flush_masked():
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(capacity=16)
    A, dt_bias, S0, seq = _mamba2_case(sh, base.cfg_seed, 0, 11)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    seq64 = [mamba2_step_f64(s) for s in seq]
    _, Ss_ref = o_m2.run_standard(S0.astype(np.float64), seq64, dt_bias.astype(np.float64),
                                  A.astype(np.float64), sh.ngroups)
    for st in seq:
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
    mask = dev_i32(np.array([1, 0, 1, 0]))
    before = state0.clone()
    rd.replay_flush(dims, state0, ring, mask)
    got = state0.cpu().numpy()
    for b in (0, 2):
        assert rel_err(got[b], Ss_ref[-1][b]) <= S_TOL
    for b in (1, 3):
        assert torch.equal(state0[b], before[b])
    assert ring.count.cpu().tolist() == [0, 11, 0, 11]
    assert ring.head.cpu().tolist() == [11, 0, 11, 0]


def _spec_inputs(sh, seed, cfg_id, rounds):
    out = [synth.mamba2_step_inputs(sh, seed, cfg_id, r) for r in range(rounds)]
    if sh.T == 1:   # the generator drops the draft axis at T = 1
        out = [{k_: v_[:, None] for k_, v_ in st.items()} for st in out]
    return out


@pytest.mark.parametrize("d,G,L,T", [(64, 1, 16, 4), (64, 2, 8, 2), (128, 4, 16, 3), (64, 1, 8, 4),
                                     (64, 2, 32, 8), (128, 1, 20, 5), (64, 4, 12, 6),
                                     (64, 1, 2, 1)])  # L = 2T: every round with committed entries folds
def test_replay_verify_rollback_small(d, G, L, T):
    """Speculative rounds: every draft's y (rejected included) against the
    per-draft snapshot semantics; pointers and early-flush flags bit-exact; the
    committed state after a final flush."""
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=6, head_dim=d, ngroups=G, capacity=L, T=T)
    seed, R = base.cfg_seed, 30
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    rounds = _spec_inputs(sh, seed, 2, R)
    acc = synth.accept_draws(seed, 2, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, sh.head_dim, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(sh.batch)]
    for r, st in enumerate(rounds):
        rd.replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                           dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y,
                           flushed)
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), G, acc[r])
        e = rel_err(y.cpu().numpy(), y_ref)
        assert e <= Y_TOL, (r, e)
        fl = flushed.cpu().numpy()
        hd, ct, pd = ring.head.cpu().numpy(), ring.count.cpu().numpy(), ring.pending.cpu().numpy()
        for b in range(sh.batch):
            c0, f, h_after, c_after, _ = scheds[b][r]
            assert (bool(fl[b]), hd[b], ct[b], pd[b]) == (f, h_after, c_after, T), (r, b)
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
        assert ring.count.cpu().tolist() == [scheds[b][r][4] for b in range(sh.batch)]
        assert torch.all(ring.pending == 0)
    assert int(ring.err.item()) == 0
    rd.replay_flush(dims, state0, ring)
    es = rel_err(state0.cpu().numpy(), S)
    assert es <= S_TOL, es


def test_pointer_anomalies_are_clamped_and_flagged():
    sh = synth.WORKLOADS[2].shape.with_(batch=4, capacity=16, T=4)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    A, dt_bias = synth.mamba2_head_params(sh, 1, 2)
    state0 = dev_f32(synth.state0(sh, 1, 2))
    st = synth.mamba2_step_inputs(sh, 1, 2, 0)
    y = torch.empty(sh.batch, 4, sh.nheads, sh.head_dim, device="cuda")
    rd.replay_verify_T(dims, 4, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                       dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
    rd.replay_rollback(dims, ring, dev_i32(np.array([9, -1, 4, 2])))
    assert int(ring.err.item()) & 2
    assert ring.count.cpu().tolist() == [4, 0, 4, 2]
    ring.err.zero_()
    ring.set_pointers(count=[40, 3, -2, 1])                   # corrupt count
    rd.replay_verify_T(dims, 4, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                       dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
    torch.cuda.synchronize()
    assert int(ring.err.item()) & 1
    assert torch.isfinite(y).all()
    rd.rssm_ring_reset(dims, ring)
    assert torch.all(ring.count == 0) and int(ring.err.item()) == 0


def test_ring_pointers_view():
    """rssm_ring_pointers: the int32 [B] view of the pointer words, through a slot
    map (padding and out-of-pool entries read -1, the latter flagged), each output
    optional, and a request whose head records disagree flagged as diverged."""
    sh = synth.WORKLOADS[2].shape.with_(batch=4, nheads=4, capacity=16, T=4)
    rows = 6
    dims = _dims(sh)
    ring = rd.Ring(dims, rows=rows)
    ring.set_pointers(head=[1, 2, 3, 4, 5, 15], count=[0, 7, 12, 1, 3, 9], pending=[0, 0, 4, 0, 2, 1])
    hd, ct, pd = (torch.full((4,), 99, dtype=torch.int32, device="cuda") for _ in range(3))
    ring.use_slots(dev_i32(np.array([5, -1, 2, 9])))
    rd.rssm_ring_pointers(dims, ring, hd, ct, pd)
    assert hd.cpu().tolist() == [15, -1, 3, -1]
    assert ct.cpu().tolist() == [9, -1, 12, -1]
    assert pd.cpu().tolist() == [1, -1, 4, -1]
    assert int(ring.err.item()) == 8                      # slot 9 is outside the pool
    ct.fill_(99)
    rd.rssm_ring_pointers(dims, ring, None, ct, None)      # outputs are optional
    assert ct.cpu().tolist() == [9, -1, 12, -1]
    ring.err.zero_()
    ring.use_slots(None)
    assert ring.count.cpu().tolist() == [0, 7, 12, 1, 3, 9]  # every pool row
    assert int(ring.err.item()) == 0 and ring.copies_agree()
    ring.meta.view(torch.int64)[4, 3, 0] += 1              # head 3 of row 4 moved alone
    assert ring.head.cpu().tolist() == [1, 2, 3, 4, 5, 15]  # fields from head 0's record
    assert int(ring.err.item()) == 16 and not ring.copies_agree()


def test_gdn_decode_step_small():
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=4, T=1)
    seed = base.cfg_seed
    S0 = synth.state0(sh, seed, 4)
    dims = _dims(sh)
    state = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    S = S0.astype(np.float64)
    for t in range(12):
        st = synth.gdn_round_inputs(sh, seed, 4, t)
        sq = {k: v[:, 0] for k, v in st.items()}
        rd.gdn_decode_step(dims, state, dev_bf16(sq["v"]), dev_bf16(sq["k"]), dev_bf16(sq["q"]),
                           dev_f32(sq["g"]), dev_f32(sq["beta"]), y)
        s64 = gdn_step_f64(sq)
        S, y_ref = o_gdn.householder_step(S, s64["v"], s64["k"], s64["q"], s64["g"], s64["beta"],
                                          sh.ngroups)
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, t
    assert rel_err(state.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("d,G,L,T", [(128, 32, 16, 4), (64, 8, 8, 2), (128, 16, 16, 1),
                                     (64, 8, 32, 8), (128, 32, 24, 5), (64, 4, 14, 7), (128, 8, 32, 3),
                                     (128, 32, 32, 8)])
def test_gdn_replay_verify_small(d, G, L, T):
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=3, head_dim=d, ngroups=G, capacity=L, T=T)
    seed, R = base.cfg_seed, 30
    S0 = synth.state0(sh, seed, 4)
    acc = synth.accept_draws(seed, 4, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, sh.head_dim, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    reqs = [o_gdn.GDNReplayRequest(S0[b].astype(np.float64), L, G) for b in range(sh.batch)]
    for r in range(R):
        st = synth.gdn_round_inputs(sh, seed, 4, r)
        s64 = gdn_step_f64(st)
        head_before = ring.head.cpu().numpy().copy()
        count_before = ring.count.cpu().numpy().copy()
        rd.gdn_replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                               dev_bf16(st["q"]), dev_f32(st["g"]), dev_f32(st["beta"]), y, flushed)
        y_ref, S = o_gdn.spec_round_snapshot(S, s64, G, acc[r])
        e = rel_err(y.cpu().numpy(), y_ref)
        assert e <= Y_TOL, (r, e)
        ring_u = ring.entries().cpu().numpy()
        for b in range(sh.batch):
            yb, ub, fb = reqs[b].verify_round(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b],
                                              s64["beta"][b])
            assert bool(flushed[b].item()) == fb
            assert (ring.head[b].item(), ring.count[b].item()) == (reqs[b].head, reqs[b].count)
            slots = [(head_before[b] + count_before[b] + s) % L for s in range(T)]
            assert rel_err(ring_u[b][:, slots].transpose(1, 0, 2), ub) <= Y_TOL
            reqs[b].commit(int(acc[r, b]))
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
    assert int(ring.err.item()) == 0
    rd.gdn_replay_flush(dims, state0, ring)
    es = rel_err(state0.cpu().numpy(), S)
    assert es <= S_TOL, es


@pytest.mark.parametrize("d,G,L", [(128, 32, 16), (64, 8, 8), (128, 16, 5), (64, 4, 32), (64, 8, 1), (128, 32, 2),
                                    (128, 32, 24), (128, 8, 32)])
def test_gdn_replay_append_decode_small(d, G, L):
    """GDN standard decode through the ring: y every step, flush flags, pointers
    and the checkpoint at every flush against the oracle's flush-when-full
    request model; the committed corrections in the ring against it too."""
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=3, head_dim=d, ngroups=G, capacity=L, T=1)
    seed, steps = base.cfg_seed, 2 * L + 5
    S0 = synth.state0(sh, seed, 4)
    dims = _dims(sh)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    reqs = [o_gdn.GDNReplayRequest(S0[b].astype(np.float64), L, G) for b in range(sh.batch)]
    for t in range(steps):
        st = synth.gdn_round_inputs(sh, seed, 4, t)
        sq = {k_: np.ascontiguousarray(v_[:, 0]) for k_, v_ in st.items()}
        s64 = gdn_step_f64(sq)
        rd.gdn_replay_append_decode(dims, state0, ring, dev_bf16(sq["v"]), dev_bf16(sq["k"]), dev_bf16(sq["q"]),
                                    dev_f32(sq["g"]), dev_f32(sq["beta"]), y, flushed)
        S, y_rec = o_gdn.householder_step(S, s64["v"], s64["k"], s64["q"], s64["g"], s64["beta"], G)
        assert rel_err(y.cpu().numpy(), y_rec) <= Y_TOL, t
        for b in range(sh.batch):
            yb, fb = reqs[b].decode_step(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b], s64["beta"][b])
            assert bool(flushed[b].item()) == fb, (t, b)
            assert (ring.head[b].item(), ring.count[b].item(), ring.pending[b].item()) == \
                (reqs[b].head, reqs[b].count, 0), (t, b)
            if fb:
                assert rel_err(state0[b].cpu().numpy(), reqs[b].S0) <= S_TOL, (t, b)
        assert ring.copies_agree(), t
    ring_u = ring.entries().cpu().numpy()
    for b in range(sh.batch):
        for j in range(reqs[b].count):
            sl = (reqs[b].head + j) % L
            assert rel_err(ring_u[b][:, sl], reqs[b].ring[sl].u) <= Y_TOL, (b, j)
    assert int(ring.err.item()) == 0
    rd.gdn_replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("d,G,L,H,n", [(64, 1, 8, 8, 128), (64, 2, 5, 8, 128), (128, 4, 16, 8, 128),
                                       (64, 8, 24, 8, 128), (128, 2, 32, 8, 128), (64, 2, 8, 6, 128),
                                       (128, 4, 4, 12, 128), (64, 2, 8, 8, 64), (128, 8, 16, 8, 64),
                                       (64, 4, 8, 8, 256), (128, 1, 32, 8, 256), (64, 2, 6, 6, 256)])
def test_replay_append_decode_conv_small(d, G, L, H, n):
    """Fused front-end: conv1d + SiLU over the xBC channels gives v, k, q (bf16),
    then the ReplaySSM step.  y every step against the oracle conv -> bf16 ->
    recurrence; the written conv state bit-exact every step (buffers swapped);
    the checkpoint at every flush.  Three heads per group (H = 6, G = 2 and
    H = 12, G = 4) split a group's B and C conv states in unequal shares; at
    n = 256 a thread takes four conv channels instead of two."""
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(head_dim=d, ngroups=G, capacity=L, nheads=H, state_dim=n)
    B, H, N = sh.batch, sh.nheads, sh.state_dim
    C = H * d + 2 * G * N
    seed, steps = base.cfg_seed, 2 * L + 3
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = synth.state0(sh, seed, 0)
    cs_bits, w_bits = synth.conv_layer(B, C, 4, seed, 0)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    cs = [dev_bf16(cs_bits), dev_bf16(cs_bits)]
    w = dev_bf16(w_bits)
    y = torch.empty(B, H, d, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    cs64 = synth.bf16_bits_to_f64(cs_bits)
    W64 = synth.bf16_bits_to_f64(w_bits)
    for t in range(steps):
        x_bits = synth.conv_step_input(B, C, seed, 0, t)
        dt = synth.mamba2_step_inputs(sh, seed, 0, t)["dt"]
        cin, cout = cs[t % 2], cs[(t + 1) % 2]
        rd.replay_append_decode_conv(dims, state0, ring, cin, cout, dev_bf16(x_bits), w, dev_f32(dt),
                                     dev_f32(dt_bias), dev_f32(A), y, flushed)
        out, cs64 = o_conv.update(cs64, synth.bf16_bits_to_f64(x_bits), W64)
        v, k, q = o_conv.split_xbc(o_conv.round_bf16(out), H, d, G, N)
        delta, a = o_m2.step_size_and_decay(dt.astype(np.float64), dt_bias.astype(np.float64),
                                            A.astype(np.float64))
        S, y_ref = o_m2.standard_step(S, v, k, q, delta, a, G)
        e = rel_err(y.cpu().numpy(), y_ref)
        assert e <= Y_TOL, (t, e)
        got = synth.bf16_bits_to_f64(cout.view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.array_equal(got, cs64), t
        fl = (t + 1) % L == 0
        assert bool(torch.all(flushed == int(fl))), t
        if fl:
            assert rel_err(state0.cpu().numpy(), S) <= S_TOL, t
    assert int(ring.err.item()) == 0


def test_single_request_single_head():
    """The smallest batch: one request, one head, one group; append-decode over
    three ring cycles, then verify rounds with rollback, against the oracle."""
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(batch=1, nheads=1, ngroups=1, capacity=4)
    seed, steps = base.cfg_seed, 13
    A, dt_bias, S0, seq = _mamba2_case(sh, seed, 0, steps)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(1, 1, sh.head_dim, device="cuda")
    ys_ref, Ss_ref = o_m2.run_standard(S0.astype(np.float64), [mamba2_step_f64(st) for st in seq],
                                       dt_bias.astype(np.float64), A.astype(np.float64), 1)
    for t, st in enumerate(seq):
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                                dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        assert rel_err(y.cpu().numpy(), ys_ref[t]) <= Y_TOL, t
    assert ring.count.cpu().tolist() == [steps % 4]
    S = Ss_ref[-1]
    T = 2
    shv = sh.with_(T=T)
    acc = np.array([[2], [0], [1], [2], [1]], dtype=np.int32)
    y2 = torch.empty(1, T, 1, sh.head_dim, device="cuda")
    for r in range(len(acc)):
        st = synth.mamba2_step_inputs(shv, seed, 0, 100 + r)
        rd.replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                           dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y2)
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), 1, acc[r])
        assert rel_err(y2.cpu().numpy(), y_ref) <= Y_TOL, r
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL
    assert int(ring.err.item()) == 0


@pytest.mark.parametrize("B,C", [(1, 2), (3, 70), (5, 3070)])
def test_causal_conv1d_update_ragged(B, C):
    """Channel counts that are even but not a multiple of four, and grids whose last
    work-group is partly empty: state shift bit for bit, outputs to 1e-5."""
    st_bits, w_bits = synth.conv_layer(B, C, 4, 777, 1)
    state = dev_bf16(st_bits)
    w = dev_bf16(w_bits)
    out = torch.full((B, C), float("nan"), device="cuda")
    ref_state = synth.bf16_bits_to_f64(st_bits)
    W = synth.bf16_bits_to_f64(w_bits)
    for t in range(3):
        x_bits = synth.conv_step_input(B, C, 777, 1, t)
        rd.causal_conv1d_update(state, dev_bf16(x_bits), w, out)
        o_ref, ref_state = o_conv.update(ref_state, synth.bf16_bits_to_f64(x_bits), W)
        assert rel_err(out.cpu().numpy(), o_ref) <= 1e-5
        got_bits = state.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(synth.bf16_bits_to_f64(got_bits), ref_state)


def test_causal_conv1d_update_config1_size():
    wl = synth.WORKLOADS[1]
    B, C = wl.shape.batch, wl.conv_channels
    st_bits, w_bits = synth.conv_layer(B, C, 4, wl.cfg_seed, 1)
    state = dev_bf16(st_bits)
    w = dev_bf16(w_bits)
    out = torch.empty(B, C, device="cuda")
    ref_state = synth.bf16_bits_to_f64(st_bits)
    W = synth.bf16_bits_to_f64(w_bits)
    for t in range(6):
        x_bits = synth.conv_step_input(B, C, wl.cfg_seed, 1, t)
        rd.causal_conv1d_update(state, dev_bf16(x_bits), w, out)
        o_ref, ref_state = o_conv.update(ref_state, synth.bf16_bits_to_f64(x_bits), W)
        assert rel_err(out.cpu().numpy(), o_ref) <= 1e-5
        got_bits = state.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(synth.bf16_bits_to_f64(got_bits), ref_state)
