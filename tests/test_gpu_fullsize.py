"""GPU parity at the full workload sizes, in the launch configuration bench.py
times, over the full step/round counts.

The oracle follows sampled (request, head) pairs, each as its own pseudo-request
(heads and requests are independent, so this is an exact check of those outputs),
over the whole run; over the first 2L steps (8 verify rounds) it also follows two
heads of every request, the heads rotating so that every head is covered, which
includes every request's first flush; ring pointers and flush flags are compared
for every request at every step.  Step
inputs cycle through a pool of seeded synthetic steps (the work does not depend on
the values).  Bars: y 1e-3 and fp32 state 1e-4 (tests/util.rel_err); integers
bit-exact.
"""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import conv1d as o_conv
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from oracle import replay as o_rep
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, every_request_pairs, pair_index, sample_pairs
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4
NPAIRS = 16


def _f64(bits):
    return synth.bf16_bits_to_f64(bits)


def _pairs_arrays(pairs, H, G):
    bi = np.array([b for b, _ in pairs])
    hi = np.array([h for _, h in pairs])
    return bi, hi, hi // (H // G)


def _sub_step(st, bi, hi, gi, spec):
    """Sampled pairs of one step (or round) as float64 pseudo-requests with one head."""
    if not spec:
        return {"v": _f64(st["v"][bi, hi])[:, None], "k": _f64(st["k"][bi, gi])[:, None],
                "q": _f64(st["q"][bi, gi])[:, None], "dt": st["dt"][bi, hi].astype(np.float64)[:, None]}
    return {"v": _f64(st["v"][bi, :, hi])[:, :, None], "k": _f64(st["k"][bi, :, gi])[:, :, None],
            "q": _f64(st["q"][bi, :, gi])[:, :, None],
            "dt": st["dt"][bi, :, hi].astype(np.float64)[:, :, None]}


def _dev_step(st):
    return {k: (dev_bf16(v) if v.dtype == np.uint16 else dev_f32(v)) for k, v in st.items()}


class _EveryRequest:
    """The early-window check: the oracle over two heads of every request."""

    def __init__(self, B, H, G, S0, pool, window, spec, gdn=False, A=None, bias=None):
        self.pairs = every_request_pairs(B, H)
        self.bi, self.hi, self.gi = _pairs_arrays(self.pairs, H, G)
        self.tb, self.th = pair_index(self.pairs)
        self.window, self.spec, self.gdn, self.P = window, spec, gdn, len(pool)
        bi, hi, gi = self.bi, self.hi, self.gi
        pool = pool[:min(window, len(pool))]  # step t uses pool[t % P], as on the device
        if gdn:
            self.sub = [{"v": _f64(st["v"][bi, :, hi])[:, :, None], "k": _f64(st["k"][bi, :, gi])[:, :, None],
                         "q": _f64(st["q"][bi, :, gi])[:, :, None],
                         "g": st["g"][bi, :, hi].astype(np.float64)[:, :, None],
                         "beta": st["beta"][bi, :, hi].astype(np.float64)[:, :, None]} for st in pool]
        else:
            self.sub = [_sub_step(st, bi, hi, gi, spec) for st in pool]
            self.A = A[hi].astype(np.float64)[:, None]
            self.bias = bias[hi].astype(np.float64)[:, None]
        self.S = S0[bi, hi].astype(np.float64)[:, None]

    def step(self, t, y, state0, flushed):
        """Standard decode step t (< window): y every step, S_0 on a flush step."""
        st = self.sub[t % self.P]
        delta, a = o_m2.step_size_and_decay(st["dt"], self.bias, self.A)
        self.S, y_ref = o_m2.standard_step(self.S, st["v"], st["k"], st["q"], delta, a, 1)
        e = rel_err(y[self.tb, self.th].cpu().numpy(), y_ref[:, 0])
        assert e <= Y_TOL, ("every request", t, e)
        fl = flushed.cpu().numpy()[self.bi].astype(bool)
        if fl.any():
            e = rel_err(state0[self.tb, self.th].cpu().numpy()[fl], self.S[fl, 0])
            assert e <= S_TOL, ("every request", t, e)

    def round(self, r, acc, y, state0, flushed):
        """Verify round r (< window): every draft's y; for the requests that flushed
        this round, S_0 equals the committed state at the round's start."""
        before = self.S
        if self.gdn:
            y_ref, self.S = o_gdn.spec_round_snapshot(self.S, self.sub[r % self.P], 1, acc[r, self.bi])
        else:
            y_ref, self.S = o_m2.spec_round_snapshot(self.S, self.sub[r % self.P], self.bias, self.A, 1,
                                                     acc[r, self.bi])
        e = rel_err(y[self.tb, :, self.th].cpu().numpy(), y_ref[:, :, 0])
        assert e <= Y_TOL, ("every request", r, e)
        fl = flushed.cpu().numpy()[self.bi].astype(bool)
        if fl.any():
            got = state0[self.tb, self.th].cpu().numpy()[fl]
            e = rel_err(got, before[fl, 0])
            assert e <= S_TOL, ("every request", r, e)


def _mamba2_setup(wl, shape, pool_size, spec=False):
    sh, seed, cid = shape, wl.cfg_seed, wl.cfg_id
    A, bias = synth.mamba2_head_params(sh, seed, cid)
    S0 = synth.state0(sh, seed, cid)
    pool = [synth.mamba2_step_inputs(sh, seed, cid, p) for p in range(pool_size)]
    return A, bias, S0, pool


def test_config1_standard_and_replay_full():
    """B=256, H=32, d=64, n=128, G=8, L=16, 1024 steps (64 flushes): the standard
    step and ReplaySSM append-decode side by side from the same checkpoint, plus
    the causal conv1d update over the same 1024 steps."""
    wl = synth.WORKLOADS[1]
    sh = wl.shape
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    A, bias, S0, pool = _mamba2_setup(wl, sh, 64)
    pairs = sample_pairs(B, H, NPAIRS, seed=11)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims)
    state_r = dev_f32(S0)
    state_s = state_r.clone()
    y_r = torch.empty(B, H, D, device="cuda")
    y_s = torch.empty(B, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    dpool = [_dev_step(st) for st in pool]
    subpool = [_sub_step(st, bi, hi, gi, False) for st in pool]
    Ab, biasb = dev_f32(A), dev_f32(bias)
    S = S0[bi, hi].astype(np.float64)[:, None]
    A_sub, bias_sub = A[hi].astype(np.float64)[:, None], bias[hi].astype(np.float64)[:, None]
    sched = o_rep.pointer_schedule_standard(L, wl.steps)
    early = _EveryRequest(B, H, G, S0, pool, 2 * L, False, A=A, bias=bias)
    # conv1d state update at the same size
    C = wl.conv_channels
    cst, cw = synth.conv_layer(B, C, 4, wl.cfg_seed, 1)
    conv_state, conv_w = dev_bf16(cst), dev_bf16(cw)
    conv_out = torch.empty(B, C, device="cuda")
    conv_ref_state, W64 = _f64(cst), _f64(cw)
    xs = [synth.conv_step_input(B, C, wl.cfg_seed, 1, p) for p in range(64)]
    dxs = [dev_bf16(x) for x in xs]
    worst = [0.0, 0.0, 0.0]
    for t in range(wl.steps):
        ip = dpool[t % 64]
        rd.ssm_decode_step(dims, state_s, ip["v"], ip["k"], ip["q"], ip["dt"], biasb, Ab, y_s)
        rd.replay_append_decode(dims, state_r, ring, ip["v"], ip["k"], ip["q"], ip["dt"], biasb, Ab,
                                y_r, flushed)
        rd.causal_conv1d_update(conv_state, dxs[t % 64], conv_w, conv_out)
        st = subpool[t % 64]
        delta, a = o_m2.step_size_and_decay(st["dt"], bias_sub, A_sub)
        S, y_ref = o_m2.standard_step(S, st["v"], st["k"], st["q"], delta, a, 1)
        er = rel_err(y_r[tb, th].cpu().numpy(), y_ref[:, 0])
        es = rel_err(y_s[tb, th].cpu().numpy(), y_ref[:, 0])
        assert er <= Y_TOL and es <= Y_TOL, (t, er, es)
        worst[0] = max(worst[0], er, es)
        if t < early.window:
            early.step(t, y_r, state_r, flushed)
        head, count, fl = sched[t]
        assert bool(torch.all(ring.head == head)) and bool(torch.all(ring.count == count)), t
        assert ring.copies_agree(), t
        assert bool(torch.all(flushed == int(fl))), t
        if fl:
            e = rel_err(state_r[tb, th].cpu().numpy(), S[:, 0])
            assert e <= S_TOL, (t, e)
            worst[1] = max(worst[1], e)
        o_ref, conv_ref_state = o_conv.update(conv_ref_state, _f64(xs[t % 64]), W64)
        if t % 128 == 127:
            assert rel_err(conv_out.cpu().numpy(), o_ref) <= 1e-5, t
    e = rel_err(state_s[tb, th].cpu().numpy(), S[:, 0])
    assert e <= S_TOL
    got_bits = conv_state.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(_f64(got_bits), conv_ref_state)
    assert int(ring.err.item()) == 0


def test_config2_speculative_verify_full():
    """B=512, H=32, d=64, n=128, G=1, L=16, T=4, 256 verify rounds with random
    acceptance and rollback by pointer."""
    wl = synth.WORKLOADS[2]
    sh = wl.shape
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    A, bias, S0, pool = _mamba2_setup(wl, sh, 32)
    acc = synth.accept_draws(wl.cfg_seed, 2, wl.steps, B, T)
    pairs = sample_pairs(B, H, NPAIRS, seed=22)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(B, T, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    dpool = [_dev_step(st) for st in pool]
    subpool = [_sub_step(st, bi, hi, gi, True) for st in pool]
    Ab, biasb = dev_f32(A), dev_f32(bias)
    S = S0[bi, hi].astype(np.float64)[:, None]
    A_sub, bias_sub = A[hi].astype(np.float64)[:, None], bias[hi].astype(np.float64)[:, None]
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(B)]
    sched_arr = np.array(scheds)            # [B, R, 5]
    dacc = [dev_i32(acc[r]) for r in range(wl.steps)]
    early = _EveryRequest(B, H, G, S0, pool, 8, True, A=A, bias=bias)
    for r in range(wl.steps):
        ip = dpool[r % 32]
        rd.replay_verify_T(dims, T, state0, ring, ip["v"], ip["k"], ip["q"], ip["dt"], biasb, Ab, y,
                           flushed)
        y_ref, S = o_m2.spec_round_snapshot(S, subpool[r % 32], bias_sub, A_sub, 1, acc[r, bi])
        e = rel_err(y[tb, :, th].cpu().numpy(), y_ref[:, :, 0])
        assert e <= Y_TOL, (r, e)
        if r < early.window:
            early.round(r, acc, y, state0, flushed)
        assert np.array_equal(flushed.cpu().numpy(), sched_arr[:, r, 1].astype(np.int32)), r
        assert np.array_equal(ring.head.cpu().numpy(), sched_arr[:, r, 2]), r
        assert np.array_equal(ring.count.cpu().numpy(), sched_arr[:, r, 3]), r
        rd.replay_rollback(dims, ring, dacc[r])
        assert np.array_equal(ring.count.cpu().numpy(), sched_arr[:, r, 4]), r
        assert ring.copies_agree(), r
    assert int(ring.err.item()) == 0
    rd.replay_flush(dims, state0, ring)
    e = rel_err(state0[tb, th].cpu().numpy(), S[:, 0])
    assert e <= S_TOL, e


@pytest.mark.parametrize("L", [4, 8, 16, 32])
def test_config3_capacity_sweep_full(L):
    """B=256, H=128, d=64, n=128, G=8, 2048 steps at ring capacity L: sampled y
    every step, every request's pointers and flush flag every step, the sampled
    checkpoint at every flush."""
    wl = synth.WORKLOADS[3]
    sh = wl.shape.with_(capacity=L)
    B, H, D, N, G = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups
    A, bias, S0, pool = _mamba2_setup(wl, sh, 32)
    pairs = sample_pairs(B, H, NPAIRS, seed=33 + L)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(B, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    dpool = [_dev_step(st) for st in pool]
    subpool = [_sub_step(st, bi, hi, gi, False) for st in pool]
    Ab, biasb = dev_f32(A), dev_f32(bias)
    S = S0[bi, hi].astype(np.float64)[:, None]
    A_sub, bias_sub = A[hi].astype(np.float64)[:, None], bias[hi].astype(np.float64)[:, None]
    sched = o_rep.pointer_schedule_standard(L, wl.steps)
    early = _EveryRequest(B, H, G, S0, pool, 2 * L, False, A=A, bias=bias)
    for t in range(wl.steps):
        ip = dpool[t % 32]
        rd.replay_append_decode(dims, state0, ring, ip["v"], ip["k"], ip["q"], ip["dt"], biasb, Ab, y,
                                flushed)
        st = subpool[t % 32]
        delta, a = o_m2.step_size_and_decay(st["dt"], bias_sub, A_sub)
        S, y_ref = o_m2.standard_step(S, st["v"], st["k"], st["q"], delta, a, 1)
        e = rel_err(y[tb, th].cpu().numpy(), y_ref[:, 0])
        assert e <= Y_TOL, (t, e)
        if t < early.window:
            early.step(t, y, state0, flushed)
        head, count, fl = sched[t]
        assert bool(torch.all(ring.head == head)) and bool(torch.all(ring.count == count)), t
        assert bool(torch.all(flushed == int(fl))), t
        if t % 64 == 0 or fl:
            assert ring.copies_agree(), t
        if fl:
            es = rel_err(state0[tb, th].cpu().numpy(), S[:, 0])
            assert es <= S_TOL, (t, es)
    assert int(ring.err.item()) == 0
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0[tb, th].cpu().numpy(), S[:, 0]) <= S_TOL


def test_config4_gdn_verify_full():
    """Gated DeltaNet B=256, H=32, d=128, n=128, G=32, L=16, T=4, 512 rounds, plus
    the standard GDN step at the same size."""
    wl = synth.WORKLOADS[4]
    sh = wl.shape
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    S0 = synth.state0(sh, wl.cfg_seed, 4)
    pool = [synth.gdn_round_inputs(sh, wl.cfg_seed, 4, p) for p in range(32)]
    acc = synth.accept_draws(wl.cfg_seed, 4, wl.steps, B, T)
    pairs = sample_pairs(B, H, NPAIRS, seed=44)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(B, T, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    dpool = [_dev_step(st) for st in pool]
    subpool = []
    for st in pool:
        subpool.append({"v": _f64(st["v"][bi, :, hi])[:, :, None], "k": _f64(st["k"][bi, :, gi])[:, :, None],
                        "q": _f64(st["q"][bi, :, gi])[:, :, None],
                        "g": st["g"][bi, :, hi].astype(np.float64)[:, :, None],
                        "beta": st["beta"][bi, :, hi].astype(np.float64)[:, :, None]})
    S = S0[bi, hi].astype(np.float64)[:, None]
    scheds = np.array([o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(B)])
    dacc = [dev_i32(acc[r]) for r in range(wl.steps)]
    early = _EveryRequest(B, H, G, S0, pool, 8, True, gdn=True)
    for r in range(wl.steps):
        ip = dpool[r % 32]
        rd.gdn_replay_verify_T(dims, T, state0, ring, ip["v"], ip["k"], ip["q"], ip["g"], ip["beta"], y,
                               flushed)
        y_ref, S = o_gdn.spec_round_snapshot(S, subpool[r % 32], 1, acc[r, bi])
        e = rel_err(y[tb, :, th].cpu().numpy(), y_ref[:, :, 0])
        assert e <= Y_TOL, (r, e)
        if r < early.window:
            early.round(r, acc, y, state0, flushed)
        assert np.array_equal(flushed.cpu().numpy(), scheds[:, r, 1].astype(np.int32)), r
        assert np.array_equal(ring.head.cpu().numpy(), scheds[:, r, 2]), r
        assert np.array_equal(ring.count.cpu().numpy(), scheds[:, r, 3]), r
        assert ring.copies_agree(), r
        rd.replay_rollback(dims, ring, dacc[r])
    assert int(ring.err.item()) == 0
    rd.gdn_replay_flush(dims, state0, ring)
    assert rel_err(state0[tb, th].cpu().numpy(), S[:, 0]) <= S_TOL
    # standard GDN step at full size, continuing from the flushed checkpoint
    yd = torch.empty(B, H, D, device="cuda")
    for t in range(8):
        st = pool[t]
        sq = {k: np.ascontiguousarray(v[:, 0]) for k, v in st.items()}
        rd.gdn_decode_step(dims, state0, dev_bf16(sq["v"]), dev_bf16(sq["k"]), dev_bf16(sq["q"]),
                           dev_f32(sq["g"]), dev_f32(sq["beta"]), yd)
        sub = {"v": _f64(sq["v"][bi, hi])[:, None], "k": _f64(sq["k"][bi, gi])[:, None],
               "q": _f64(sq["q"][bi, gi])[:, None], "g": sq["g"][bi, hi].astype(np.float64)[:, None],
               "beta": sq["beta"][bi, hi].astype(np.float64)[:, None]}
        S, y_ref = o_gdn.householder_step(S, sub["v"], sub["k"], sub["q"], sub["g"], sub["beta"], 1)
        assert rel_err(yd[tb, th].cpu().numpy(), y_ref[:, 0]) <= Y_TOL, t
    assert rel_err(state0[tb, th].cpu().numpy(), S[:, 0]) <= S_TOL


@pytest.mark.parametrize("gdn", [False, True])
def test_snapshot_route_full(gdn):
    """The per-draft snapshot route at the speculative workloads' full sizes
    (Mamba-2 B=512, H=32, d=64, G=1; GDN B=256, H=32, d=128, G=32; T=4, T + 1
    slots per request), 32 rounds with seeded acceptance and the device-side
    commit: sampled y every round, the committed snapshot of the sampled pairs
    every 8 rounds, every request's slot index every round."""
    cid = 4 if gdn else 2
    wl = synth.WORKLOADS[cid]
    sh = wl.shape
    B, H, D, N, G, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.T
    P, R = T + 1, 32
    S0 = synth.state0(sh, wl.cfg_seed, cid)
    acc = synth.accept_draws(wl.cfg_seed, cid, R, B, T)
    pairs = sample_pairs(B, H, NPAIRS, seed=55 + cid)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    dims = rd.Dims(B, H, D, N, G, sh.capacity)
    pool_d = torch.empty(B, P, H, D, N, device="cuda")
    pool_d[:, 0] = dev_f32(S0)
    del S0
    slot = torch.zeros(B, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty(B, T, H, D, device="cuda")
    S = pool_d[tb, 0, th].cpu().numpy().astype(np.float64)[:, None]
    if not gdn:
        A, bias = synth.mamba2_head_params(sh, wl.cfg_seed, cid)
        Ab, biasb = dev_f32(A), dev_f32(bias)
        A_sub, bias_sub = A[hi].astype(np.float64)[:, None], bias[hi].astype(np.float64)[:, None]
    cur = np.zeros(B, np.int64)
    for r in range(R):
        if gdn:
            st = synth.gdn_round_inputs(sh, wl.cfg_seed, cid, r % 8)
            ip = _dev_step(st)
            rd.gdn_snapshot_verify_T(dims, T, pool_d, slot, ip["v"], ip["k"], ip["q"], ip["g"], ip["beta"], y, err)
            sub = {"v": _f64(st["v"][bi, :, hi])[:, :, None], "k": _f64(st["k"][bi, :, gi])[:, :, None],
                   "q": _f64(st["q"][bi, :, gi])[:, :, None],
                   "g": st["g"][bi, :, hi].astype(np.float64)[:, :, None],
                   "beta": st["beta"][bi, :, hi].astype(np.float64)[:, :, None]}
            y_ref, S = o_gdn.spec_round_snapshot(S, sub, 1, acc[r, bi])
        else:
            st = synth.mamba2_step_inputs(sh, wl.cfg_seed, cid, r % 8)
            ip = _dev_step(st)
            rd.ssm_snapshot_verify_T(dims, T, pool_d, slot, ip["v"], ip["k"], ip["q"], ip["dt"], biasb, Ab, y,
                                     err)
            y_ref, S = o_m2.spec_round_snapshot(S, _sub_step(st, bi, hi, gi, True), bias_sub, A_sub, 1,
                                                acc[r, bi])
        e = rel_err(y[tb, :, th].cpu().numpy(), y_ref[:, :, 0])
        assert e <= Y_TOL, (r, e)
        rd.snapshot_commit(T, P, slot, dev_i32(acc[r]), err)
        cur = (cur + acc[r]) % P
        assert np.array_equal(slot.cpu().numpy(), cur), r
        if r % 8 == 7:
            got = pool_d[tb, slot[tb].long(), th].cpu().numpy()
            es = rel_err(got, S[:, 0])
            assert es <= S_TOL, (r, es)
    assert int(err.item()) == 0


def test_gdn_append_decode_full():
    """GDN standard decode through the ring at the GDN workload's size (B=256,
    H=32, d=128, G=32, L=16), 64 steps (4 flush cycles): sampled y every step and
    the sampled checkpoint at every flush against the recurrence; flush flags and
    pointers of every request every step."""
    wl = synth.WORKLOADS[4]
    sh = wl.shape.with_(T=1)
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    S0 = synth.state0(sh, wl.cfg_seed, 4)
    pool = [synth.gdn_round_inputs(sh, wl.cfg_seed, 4, p) for p in range(16)]
    pool = [{k: np.ascontiguousarray(v[:, 0]) for k, v in st.items()} for st in pool]
    pairs = sample_pairs(B, H, NPAIRS, seed=66)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(B, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    dpool = [_dev_step(st) for st in pool]
    S = S0[bi, hi].astype(np.float64)[:, None]
    del S0
    for t in range(64):
        st, ip = pool[t % 16], dpool[t % 16]
        rd.gdn_replay_append_decode(dims, state0, ring, ip["v"], ip["k"], ip["q"], ip["g"], ip["beta"], y, flushed)
        sub = {"v": _f64(st["v"][bi, hi])[:, None], "k": _f64(st["k"][bi, gi])[:, None],
               "q": _f64(st["q"][bi, gi])[:, None], "g": st["g"][bi, hi].astype(np.float64)[:, None],
               "beta": st["beta"][bi, hi].astype(np.float64)[:, None]}
        S, y_ref = o_gdn.householder_step(S, sub["v"], sub["k"], sub["q"], sub["g"], sub["beta"], 1)
        e = rel_err(y[tb, th].cpu().numpy(), y_ref[:, 0])
        assert e <= Y_TOL, (t, e)
        fl = (t + 1) % L == 0
        assert bool(torch.all(flushed == int(fl))), t
        assert bool(torch.all(ring.count == (t + 1) % L)) and bool(torch.all(ring.head == 0)), t
        if fl:
            es = rel_err(state0[tb, th].cpu().numpy(), S[:, 0])
            assert es <= S_TOL, (t, es)
    assert ring.copies_agree()
    assert int(ring.err.item()) == 0


def test_fused_front_end_full():
    """replay_append_decode_conv at the Nemotron-H-like size (B=256, H=32, d=64,
    G=8, L=16, C = H d + 2 G n = 4096 xBC channels), 48 steps (3 flushes): sampled
    y every step and the sampled checkpoint at every flush against the oracle's
    conv -> bf16 -> recurrence on those (request, head) pairs' channels; every
    request's new v and k, as cached in the ring, bit-exact against the oracle's
    conv and bf16 rounding every step but the flush steps (786,432 rounding
    decisions a step); the whole written conv state bit-exact every 8 steps."""
    wl = synth.WORKLOADS[1]
    sh = wl.shape
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    C, seed = H * D + 2 * G * N, wl.cfg_seed
    A, bias = synth.mamba2_head_params(sh, seed, 1)
    S0 = synth.state0(sh, seed, 1)
    cs_bits, w_bits = synth.conv_layer(B, C, 4, seed, 1, layer=1)
    pairs = sample_pairs(B, H, NPAIRS, seed=77)
    bi, hi, gi = _pairs_arrays(pairs, H, G)
    tb, th = pair_index(pairs)
    # the channels each pair's oracle follows: its head's x, its group's B and C
    chans = np.stack([np.concatenate([h * D + np.arange(D), H * D + g * N + np.arange(N),
                                      H * D + G * N + g * N + np.arange(N)]) for h, g in zip(hi, gi)])
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    cs = [dev_bf16(cs_bits), dev_bf16(cs_bits)]
    w = dev_bf16(w_bits)
    y = torch.empty(B, H, D, device="cuda")
    S = S0[bi, hi].astype(np.float64)[:, None]
    del S0
    cs64_all = _f64(cs_bits)
    W64 = _f64(w_bits)
    sub_state = np.stack([cs64_all[b][ch] for b, ch in zip(bi, chans)])       # [P, 320, 3]
    sub_w = np.stack([W64[ch] for ch in chans])                               # [P, 320, 4]
    Ab, biasb = dev_f32(A), dev_f32(bias)
    for t in range(48):
        x_bits = synth.conv_step_input(B, C, seed, 1, t, layer=1)
        dt = synth.mamba2_step_inputs(sh, seed, 1, t)["dt"]
        cin, cout = cs[t % 2], cs[(t + 1) % 2]
        rd.replay_append_decode_conv(dims, state0, ring, cin, cout, dev_bf16(x_bits), w, dev_f32(dt), biasb, Ab,
                                     y)
        x64 = _f64(x_bits)
        xs = np.stack([x64[b][ch] for b, ch in zip(bi, chans)])              # [P, 320]
        # per pair: the oracle conv over its own channels (each pair has its taps)
        outs, states = [], []
        for p_ in range(len(pairs)):
            o_, s_ = o_conv.update(sub_state[p_:p_ + 1], xs[p_:p_ + 1], sub_w[p_])
            outs.append(o_[0])
            states.append(s_[0])
        out = o_conv.round_bf16(np.stack(outs))
        sub_state = np.stack(states)
        v, k, q = out[:, None, :D], out[:, None, D:D + N], out[:, None, D + N:]
        delta, a = o_m2.step_size_and_decay(dt[bi, hi].astype(np.float64)[:, None],
                                            bias[hi].astype(np.float64)[:, None], A[hi].astype(np.float64)[:, None])
        S, y_ref = o_m2.standard_step(S, v, k, q, delta, a, 1)
        e = rel_err(y[tb, th].cpu().numpy(), y_ref[:, 0])
        assert e <= Y_TOL, (t, e)
        if (t + 1) % L:
            # every request's new v and k as cached in the ring: the conv's bf16
            # rounding decisions, bit for bit (entry t mod L: head stays 0)
            full = o_conv.round_bf16(o_conv.update(cs64_all, x64, W64)[0])
            v_all, k_all, _ = o_conv.split_xbc(full, H, D, G, N)
            sl = t % L
            got_v = _f64(ring.entries()[:, :, sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
            got_k = _f64(ring.k[:, :, sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
            assert np.array_equal(got_v, v_all) and np.array_equal(got_k, k_all), t
        cs64_all = np.concatenate([cs64_all[:, :, 1:], x64[:, :, None]], axis=-1)   # the state shift
        if t % 8 == 7:
            got = _f64(cout.view(torch.int16).cpu().numpy().view(np.uint16))
            assert np.array_equal(got, cs64_all), t
        if (t + 1) % L == 0:
            es = rel_err(state0[tb, th].cpu().numpy(), S[:, 0])
            assert es <= S_TOL, (t, es)
    assert int(ring.err.item()) == 0
