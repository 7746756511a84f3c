"""Gated DeltaNet at state sizes n = 64 and n = 256 (besides the n = 128 of the
GDN workload) through the C ABI, against the oracle: the standard GDN step,
ReplaySSM GDN append-decode across flushes (ring capacities 5, 16 and 32),
speculative verify with random acceptance and device-side rollback followed by
an explicit flush, and the per-draft snapshot route.  Bars as elsewhere: y
1e-3, fp32 state 1e-4, pointers and flush flags bit-exact."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import gdn as o_gdn
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4
SHAPES = [(64, 64, 4), (128, 64, 2), (64, 256, 4), (128, 256, 1)]   # (d, n, G), H = 4


def _shape(d, n, G, L, T=1, B=3, H=4):
    return synth.WORKLOADS[4].shape.with_(batch=B, nheads=H, head_dim=d, state_dim=n, ngroups=G, capacity=L, T=T)


def _dims(sh):
    return rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity)


def _step(st):
    return {k_: np.ascontiguousarray(v_[:, 0]) for k_, v_ in st.items()}


@pytest.mark.parametrize("d,n,G", SHAPES)
def test_gdn_standard_step(d, n, G):
    sh = _shape(d, n, G, 8)
    seed = synth.WORKLOADS[4].cfg_seed
    S0 = synth.state0(sh, seed, 4)
    dims = _dims(sh)
    state = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    S = S0.astype(np.float64)
    for t in range(6):
        sq = _step(synth.gdn_round_inputs(sh, seed, 4, t))
        s64 = gdn_step_f64(sq)
        rd.gdn_decode_step(dims, state, dev_bf16(sq["v"]), dev_bf16(sq["k"]), dev_bf16(sq["q"]),
                           dev_f32(sq["g"]), dev_f32(sq["beta"]), y)
        S, y_ref = o_gdn.householder_step(S, s64["v"], s64["k"], s64["q"], s64["g"], s64["beta"], G)
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, t
    assert rel_err(state.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("L", [5, 16, 32])
@pytest.mark.parametrize("d,n,G", SHAPES)
def test_gdn_append_decode_across_flushes(d, n, G, L):
    sh = _shape(d, n, G, L)
    seed, steps = synth.WORKLOADS[4].cfg_seed, 2 * L + 3
    S0 = synth.state0(sh, seed, 4)
    dims = _dims(sh)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    for t in range(steps):
        sq = _step(synth.gdn_round_inputs(sh, seed, 4, t))
        s64 = gdn_step_f64(sq)
        rd.gdn_replay_append_decode(dims, state0, ring, dev_bf16(sq["v"]), dev_bf16(sq["k"]), dev_bf16(sq["q"]),
                                    dev_f32(sq["g"]), dev_f32(sq["beta"]), y, flushed)
        S, y_ref = o_gdn.householder_step(S, s64["v"], s64["k"], s64["q"], s64["g"], s64["beta"], G)
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, t
        fl = (t + 1) % L == 0
        assert bool(torch.all(flushed == int(fl))), t
        assert ring.count.cpu().tolist() == [(t + 1) % L] * sh.batch, t
        assert ring.head.cpu().tolist() == [0] * sh.batch, t
        if fl:
            assert rel_err(state0.cpu().numpy(), S) <= S_TOL, t
    assert int(ring.err.item()) == 0 and ring.copies_agree()
    rd.gdn_replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("L,T", [(16, 4), (8, 2), (32, 3)])
@pytest.mark.parametrize("d,n,G", SHAPES)
def test_gdn_verify_rollback(d, n, G, L, T):
    sh = _shape(d, n, G, L, T=T)
    seed, R = synth.WORKLOADS[4].cfg_seed, 3 * L // T + 2
    S0 = synth.state0(sh, seed, 4)
    acc = synth.accept_draws(seed, 4, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, d, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    S = S0.astype(np.float64)
    reqs = [o_gdn.GDNReplayRequest(S0[b].astype(np.float64), L, G) for b in range(sh.batch)]
    for r in range(R):
        st = synth.gdn_round_inputs(sh, seed, 4, r)
        s64 = gdn_step_f64(st)
        rd.gdn_replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]),
                               dev_bf16(st["q"]), dev_f32(st["g"]), dev_f32(st["beta"]), y, flushed)
        y_ref, S = o_gdn.spec_round_snapshot(S, s64, G, acc[r])
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, r
        for b in range(sh.batch):
            _, _, fb = reqs[b].verify_round(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b], s64["beta"][b])
            assert bool(flushed[b].item()) == fb, (r, b)
            assert (ring.head[b].item(), ring.count[b].item(), ring.pending[b].item()) == \
                (reqs[b].head, reqs[b].count, T), (r, b)
            if fb:
                assert rel_err(state0[b].cpu().numpy(), reqs[b].S0) <= S_TOL, (r, b)
            reqs[b].commit(int(acc[r, b]))
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
    assert int(ring.err.item()) == 0 and ring.copies_agree()
    rd.gdn_replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("d,n,G", SHAPES)
def test_gdn_snapshot_route(d, n, G):
    T, P, R = 3, 5, 6
    sh = _shape(d, n, G, 8, T=T)
    seed = synth.WORKLOADS[4].cfg_seed
    B = sh.batch
    S0 = synth.state0(sh, seed, 4)
    acc = synth.accept_draws(seed, 4, R, B, T)
    pool = torch.zeros((B, P, sh.nheads, d, n), device="cuda")
    pool[:, 0] = dev_f32(S0)
    slot = dev_i32(np.zeros(B, int))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty(B, T, sh.nheads, d, device="cuda")
    dims = _dims(sh)
    S = S0.astype(np.float64)
    for r in range(R):
        st = synth.gdn_round_inputs(sh, seed, 4, r)
        rd.gdn_snapshot_verify_T(dims, T, pool, slot, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                                 dev_f32(st["g"]), dev_f32(st["beta"]), y, err)
        y_ref, S = o_gdn.spec_round_snapshot(S, gdn_step_f64(st), G, acc[r])
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, r
        rd.snapshot_commit(T, P, slot, dev_i32(acc[r]), err)
        got = pool[torch.arange(B, device="cuda"), slot.long()].cpu().numpy()
        assert rel_err(got, S) <= S_TOL, r
    assert int(err.item()) == 0
