"""Commit-and-verify (replay_commit_verify_T, gdn_replay_commit_verify_T): the
previous window's commit folded into the next verify launch.  Every round's
draft outputs against the per-draft snapshot semantics; every request's pointers
and early-flush flags bit-exact against the integer schedule (count as the
commit leaves it, then the verify's own move); the committed state after a final
device-side commit and flush; a run that mixes both call forms; accepted counts
out of range clamped and flagged as the separate commit kernel does."""
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


def _dims(sh):
    return rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity)


def _mamba2_round(sh, seed, r):
    st = synth.mamba2_step_inputs(sh, seed, 2, r)
    return {k_: v_[:, None] for k_, v_ in st.items()} if sh.T == 1 else st


@pytest.mark.parametrize("d,n,G,L,T,mixed", [(64, 128, 1, 16, 4, False), (128, 128, 2, 8, 2, False),
                                             (64, 64, 2, 12, 3, True), (64, 256, 1, 32, 5, False),
                                             (128, 128, 4, 16, 1, True)])
def test_mamba2_commit_verify(d, n, G, L, T, mixed):
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=5, head_dim=d, state_dim=n, ngroups=G, capacity=L, T=T)
    seed, R = base.cfg_seed, 3 * L // T + 3
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, d, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(sh.batch)]
    prev = dev_i32(np.zeros(sh.batch, int))      # nothing pending before the first round
    for r in range(R):
        st = _mamba2_round(sh, seed, r)
        args = (dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias),
                dev_f32(A), y, flushed)
        if mixed and r % 3 == 1:                  # the two forms interleave on one ring
            rd.replay_rollback(dims, ring, prev)
            rd.replay_verify_T(dims, T, state0, ring, *args)
        else:
            rd.replay_commit_verify_T(dims, T, state0, ring, prev, *args)
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), G, acc[r])
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, r
        fl = flushed.cpu().numpy()
        hd, ct, pd = ring.head.cpu().numpy(), ring.count.cpu().numpy(), ring.pending.cpu().numpy()
        for b in range(sh.batch):
            _, f, h_after, c_after, _ = scheds[b][r]
            assert (bool(fl[b]), hd[b], ct[b], pd[b]) == (f, h_after, c_after, T), (r, b)
        prev = dev_i32(acc[r])
    rd.replay_rollback(dims, ring, prev)
    assert ring.count.cpu().tolist() == [scheds[b][R - 1][4] for b in range(sh.batch)]
    assert int(ring.err.item()) == 0 and ring.copies_agree()
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("d,n,G,L,T", [(128, 128, 32, 16, 4), (64, 64, 8, 8, 2), (128, 256, 4, 16, 3)])
def test_gdn_commit_verify(d, n, G, L, T):
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=3, nheads=G if G >= 4 else 4, head_dim=d, state_dim=n, ngroups=G, capacity=L, T=T)
    seed, R = base.cfg_seed, 3 * L // T + 2
    S0 = synth.state0(sh, seed, 4)
    acc = synth.accept_draws(seed, 4, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, d, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(sh.batch)]
    prev = dev_i32(np.zeros(sh.batch, int))
    for r in range(R):
        st = synth.gdn_round_inputs(sh, seed, 4, r)
        rd.gdn_replay_commit_verify_T(dims, T, state0, ring, prev, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                      dev_bf16(st["q"]), dev_f32(st["g"]), dev_f32(st["beta"]), y, flushed)
        y_ref, S = o_gdn.spec_round_snapshot(S, gdn_step_f64(st), G, acc[r])
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, r
        fl = flushed.cpu().numpy()
        hd, ct = ring.head.cpu().numpy(), ring.count.cpu().numpy()
        for b in range(sh.batch):
            _, f, h_after, c_after, _ = scheds[b][r]
            assert (bool(fl[b]), hd[b], ct[b]) == (f, h_after, c_after), (r, b)
        prev = dev_i32(acc[r])
    rd.replay_rollback(dims, ring, prev)
    assert int(ring.err.item()) == 0 and ring.copies_agree()
    rd.gdn_replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL


def test_commit_verify_clamps_accepted_counts():
    sh = synth.WORKLOADS[2].shape.with_(batch=4, capacity=16, T=4)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    A, dt_bias = synth.mamba2_head_params(sh, 1, 2)
    state0 = dev_f32(synth.state0(sh, 1, 2))
    st = synth.mamba2_step_inputs(sh, 1, 2, 0)
    args = (dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias),
            dev_f32(A), torch.empty(sh.batch, 4, sh.nheads, sh.head_dim, device="cuda"))
    rd.replay_verify_T(dims, 4, state0, ring, *args)                      # 4 drafts pending everywhere
    rd.replay_commit_verify_T(dims, 4, state0, ring, dev_i32(np.array([9, -1, 4, 2])), *args)
    assert int(ring.err.item()) == 2                                       # accepted outside [0, pending]
    assert ring.count.cpu().tolist() == [4, 0, 4, 2] and torch.all(ring.pending == 4)
