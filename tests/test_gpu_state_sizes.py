"""State sizes n = 64 and n = 256 (besides the n = 128 of every workload) through
the C ABI, against the oracle: the standard Mamba-2 step, ReplaySSM
append-decode across flushes, speculative verify with random acceptance and
device-side rollback (combine on the vector ALUs for T < 3, on the matrix cores
from T = 3), and the explicit flush.  Bars as elsewhere: y 1e-3, fp32 state
1e-4, pointers and flush flags bit-exact."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import mamba2 as o_m2
from oracle import replay as o_rep
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4
SHAPES = [(64, 64, 1), (128, 64, 2), (64, 256, 2), (128, 256, 1)]   # (d, n, G)


def _shape(d, n, G, L, T=1, B=3, H=4):
    return synth.WORKLOADS[0].shape.with_(batch=B, nheads=H, head_dim=d, state_dim=n, ngroups=G, capacity=L, T=T)


def _dims(sh):
    return rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity)


@pytest.mark.parametrize("d,n,G", SHAPES)
def test_standard_step(d, n, G):
    sh = _shape(d, n, G, 8)
    seed = synth.WORKLOADS[0].cfg_seed
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = synth.state0(sh, seed, 0)
    seq = [synth.mamba2_step_inputs(sh, seed, 0, t) for t in range(6)]
    ys_ref, Ss_ref = o_m2.run_standard(S0.astype(np.float64), [mamba2_step_f64(s) for s in seq],
                                       dt_bias.astype(np.float64), A.astype(np.float64), G)
    dims = _dims(sh)
    state = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    for t, st in enumerate(seq):
        rd.ssm_decode_step(dims, state, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                           dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        assert rel_err(y.cpu().numpy(), ys_ref[t]) <= Y_TOL, t
    assert rel_err(state.cpu().numpy(), Ss_ref[-1]) <= S_TOL


@pytest.mark.parametrize("L", [5, 16, 32])
@pytest.mark.parametrize("d,n,G", SHAPES)
def test_append_decode_across_flushes(d, n, G, L):
    sh = _shape(d, n, G, L)
    seed, steps = synth.WORKLOADS[0].cfg_seed, 2 * L + 3
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = synth.state0(sh, seed, 0)
    seq = [synth.mamba2_step_inputs(sh, seed, 0, t) for t in range(steps)]
    ys_ref, Ss_ref = o_m2.run_standard(S0.astype(np.float64), [mamba2_step_f64(s) for s in seq],
                                       dt_bias.astype(np.float64), A.astype(np.float64), G)
    sched = o_rep.pointer_schedule_standard(L, steps)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    for t, st in enumerate(seq):
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                                dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y, flushed)
        assert rel_err(y.cpu().numpy(), ys_ref[t]) <= Y_TOL, t
        head, count, fl = sched[t]
        assert torch.all(ring.head == head) and torch.all(ring.count == count), t
        assert torch.all(flushed == int(fl)), t
        if fl:
            assert rel_err(state0.cpu().numpy(), Ss_ref[t]) <= S_TOL, t
    assert int(ring.err.item()) == 0
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), Ss_ref[-1]) <= S_TOL


@pytest.mark.parametrize("T,L", [(1, 4), (2, 8), (3, 8), (4, 16), (6, 16), (8, 32)])
@pytest.mark.parametrize("d,n,G", SHAPES)
def test_verify_rollback(d, n, G, T, L):
    sh = _shape(d, n, G, L, T=T)
    seed, R = synth.WORKLOADS[2].cfg_seed, 12
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, sh.batch, T)
    dims = _dims(sh)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, d, device="cuda")
    flushed = torch.zeros(sh.batch, dtype=torch.int32, device="cuda")
    scheds = np.array([o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(sh.batch)])
    S = S0.astype(np.float64)
    for r in range(R):
        st = synth.mamba2_step_inputs(sh, seed, 2, r)
        if T == 1:
            st = {k_: v_[:, None] for k_, v_ in st.items()}
        rd.replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                           dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y, flushed)
        S_before = S
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), G, acc[r])
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, r
        fl = flushed.cpu().numpy().astype(bool)
        assert np.array_equal(fl, scheds[:, r, 1].astype(bool)), r
        if fl.any():
            assert rel_err(state0.cpu().numpy()[fl], S_before[fl]) <= S_TOL, r
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
        assert np.array_equal(ring.count.cpu().numpy(), scheds[:, r, 4]), r
    assert int(ring.err.item()) == 0
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL
