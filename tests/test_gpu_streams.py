"""Two calls on disjoint buffers may run on different streams at the same time
(the library keeps no state of its own between or across calls): a Mamba-2
append-decode ring and a GDN commit-and-verify ring, each driven on its own
stream with every step's inputs and outputs in buffers of their own, launched
back to back with no host synchronisation in between, then checked step by step
against the oracle; a third stream runs the standard Mamba-2 step on a third
state alongside."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from oracle import replay as o_rep
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4


def test_independent_rings_on_concurrent_streams():
    # ring A: Mamba-2 append-decode, flush when full
    wa = synth.WORKLOADS[0]
    sha = wa.shape.with_(batch=6, nheads=8, ngroups=2, capacity=8)
    steps = 2 * sha.capacity + 5
    A, dt_bias = synth.mamba2_head_params(sha, wa.cfg_seed, 0)
    S0a = synth.state0(sha, wa.cfg_seed, 0)
    seq = [synth.mamba2_step_inputs(sha, wa.cfg_seed, 0, t) for t in range(steps)]
    dims_a = rd.Dims(sha.batch, sha.nheads, sha.head_dim, sha.state_dim, sha.ngroups, sha.capacity)
    ring_a = rd.Ring(dims_a)
    st_a = dev_f32(S0a)
    in_a = [tuple(dev_bf16(s[k]) for k in ("v", "k", "q")) + (dev_f32(s["dt"]),) for s in seq]
    y_a = [torch.empty(sha.batch, sha.nheads, sha.head_dim, device="cuda") for _ in range(steps)]
    fl_a = [torch.zeros(sha.batch, dtype=torch.int32, device="cuda") for _ in range(steps)]
    Aa, ba = dev_f32(A), dev_f32(dt_bias)

    # ring B: GDN commit-and-verify
    wb = synth.WORKLOADS[4]
    shb = wb.shape.with_(batch=4, nheads=4, ngroups=4, capacity=16, T=3)
    R = 12
    S0b = synth.state0(shb, wb.cfg_seed, 4)
    acc = synth.accept_draws(wb.cfg_seed, 4, R, shb.batch, shb.T)
    rounds = [synth.gdn_round_inputs(shb, wb.cfg_seed, 4, r) for r in range(R)]
    dims_b = rd.Dims(shb.batch, shb.nheads, shb.head_dim, shb.state_dim, shb.ngroups, shb.capacity)
    ring_b = rd.Ring(dims_b, gdn=True)
    st_b = dev_f32(S0b)
    in_b = [tuple(dev_bf16(s[k]) for k in ("v", "k", "q")) + (dev_f32(s["g"]), dev_f32(s["beta"])) for s in rounds]
    acc_b = [dev_i32(np.zeros(shb.batch, int))] + [dev_i32(acc[r]) for r in range(R)]
    y_b = [torch.empty(shb.batch, shb.T, shb.nheads, shb.head_dim, device="cuda") for _ in range(R)]
    fl_b = [torch.zeros(shb.batch, dtype=torch.int32, device="cuda") for _ in range(R)]

    # standard step on a third state
    st_c = dev_f32(S0a)
    y_c = [torch.empty(sha.batch, sha.nheads, sha.head_dim, device="cuda") for _ in range(steps)]

    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for i in range(max(steps, R)):
        if i < steps:
            v, k, q, dt = in_a[i]
            rd.replay_append_decode(dims_a, st_a, ring_a, v, k, q, dt, ba, Aa, y_a[i], fl_a[i], stream=s1)
            rd.ssm_decode_step(dims_a, st_c, v, k, q, dt, ba, Aa, y_c[i], stream=s3)
        if i < R:
            v, k, q, g, be = in_b[i]
            rd.gdn_replay_commit_verify_T(dims_b, shb.T, st_b, ring_b, acc_b[i], v, k, q, g, be, y_b[i], fl_b[i],
                                          stream=s2)
    rd.replay_rollback(dims_b, ring_b, acc_b[R], stream=s2)
    torch.cuda.synchronize()

    ys_ref, Ss_ref = o_m2.run_standard(S0a.astype(np.float64), [mamba2_step_f64(s) for s in seq],
                                       dt_bias.astype(np.float64), A.astype(np.float64), sha.ngroups)
    sched = o_rep.pointer_schedule_standard(sha.capacity, steps)
    for t in range(steps):
        assert rel_err(y_a[t].cpu().numpy(), ys_ref[t]) <= Y_TOL, t
        assert rel_err(y_c[t].cpu().numpy(), ys_ref[t]) <= Y_TOL, t
        assert torch.all(fl_a[t] == int(sched[t][2])), t
    assert int(ring_a.err.item()) == 0
    assert torch.all(ring_a.head == sched[-1][0]) and torch.all(ring_a.count == sched[-1][1])
    assert rel_err(st_c.cpu().numpy(), Ss_ref[-1]) <= S_TOL
    rd.replay_flush(dims_a, st_a, ring_a)
    assert rel_err(st_a.cpu().numpy(), Ss_ref[-1]) <= S_TOL

    S = S0b.astype(np.float64)
    scheds = [o_rep.pointer_schedule_spec(shb.capacity, shb.T, acc[:, b]) for b in range(shb.batch)]
    for r in range(R):
        y_ref, S = o_gdn.spec_round_snapshot(S, gdn_step_f64(rounds[r]), shb.ngroups, acc[r])
        assert rel_err(y_b[r].cpu().numpy(), y_ref) <= Y_TOL, r
        fl = fl_b[r].cpu().numpy()
        for b in range(shb.batch):
            assert bool(fl[b]) == scheds[b][r][1], (r, b)
    assert int(ring_b.err.item()) == 0 and ring_b.copies_agree()
    assert ring_b.count.cpu().tolist() == [scheds[b][R - 1][4] for b in range(shb.batch)]
    rd.gdn_replay_flush(dims_b, st_b, ring_b)
    assert rel_err(st_b.cpu().numpy(), S) <= S_TOL
