"""The storage-precision options (bf16 outputs, bf16 GDN corrections in the ring)
through the C ABI, against the oracle.

Bars (derived from the arithmetic; bf16 keeps 8 significand bits, so one ulp is
2^-7 to 2^-8 of the value and rounding to nearest errs by at most 2^-8 of it):
* bf16 y: the kernel rounds its fp32 y once: y within 1e-3 + 2^-8.
* bf16 GDN corrections: the oracle rounds each cached correction to bf16 from
  its float64 value, the kernel from its fp32 value; where the two straddle a
  rounding boundary (about one element in 2^16) the cached correction differs by
  one bf16 ulp, at most 2^-7 of it, and later states and outputs move by that
  much of one term: cached corrections within 2^-7, y and states within
  1e-3 + 2^-7 (with bf16 y: plus 2^-8).
The step's own outputs use its correction unrounded, on both sides."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from ssm_recurrent_decode_amd import _lib, synth
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

S_TOL = 1e-4
Y_TOL_BF16 = 1e-3 + 2.0**-8
U_TOL = 2.0**-7
GDN_TOL = 1e-3 + 2.0**-7


def _y_f64(y):
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,G,L", [(64, 1, 8), (128, 2, 5)])
def test_append_decode_bf16_y(d, G, L):
    base = synth.WORKLOADS[0]
    sh = base.shape.with_(head_dim=d, ngroups=G, capacity=L)
    seed, steps = base.cfg_seed, 2 * L + 3
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = synth.state0(sh, seed, 0)
    dims = rd.Dims(sh.batch, sh.nheads, d, sh.state_dim, G, L, flags=_lib.RSSM_F_Y_BF16)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, sh.nheads, d, dtype=torch.bfloat16, device="cuda")
    seq = [synth.mamba2_step_inputs(sh, seed, 0, t) for t in range(steps)]
    ys_ref, Ss_ref = o_m2.run_standard(S0.astype(np.float64), [mamba2_step_f64(s) for s in seq],
                                       dt_bias.astype(np.float64), A.astype(np.float64), G)
    for t, st in enumerate(seq):
        rd.replay_append_decode(dims, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                                dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        assert rel_err(_y_f64(y), ys_ref[t]) <= Y_TOL_BF16, t
        if (t + 1) % L == 0:
            assert rel_err(state0.cpu().numpy(), Ss_ref[t]) <= S_TOL, t
    assert int(ring.err.item()) == 0


@pytest.mark.parametrize("T", [4, 6])
def test_verify_bf16_y(T):
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=5, nheads=8, capacity=16, T=T)
    seed, R = base.cfg_seed, 16
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, sh.batch, T)
    dims = rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, 16, flags=_lib.RSSM_F_Y_BF16)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(sh.batch, T, sh.nheads, sh.head_dim, dtype=torch.bfloat16, device="cuda")
    S = S0.astype(np.float64)
    for r in range(R):
        st = synth.mamba2_step_inputs(sh, seed, 2, r)
        rd.replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                           dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), sh.ngroups, acc[r])
        assert rel_err(_y_f64(y), y_ref) <= Y_TOL_BF16, r
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL


@pytest.mark.parametrize("flags", [_lib.RSSM_F_U_BF16, _lib.RSSM_F_U_BF16 | _lib.RSSM_F_Y_BF16])
@pytest.mark.parametrize("d,G,L,T", [(128, 32, 16, 4), (64, 8, 8, 2)])
def test_gdn_verify_bf16_ring(flags, d, G, L, T):
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=3, head_dim=d, ngroups=G, capacity=L, T=T)
    seed, R = base.cfg_seed, 20
    S0 = synth.state0(sh, seed, 4)
    acc = synth.accept_draws(seed, 4, R, sh.batch, T)
    dims = rd.Dims(sh.batch, sh.nheads, d, sh.state_dim, G, L, flags=flags)
    ring = rd.Ring(dims, gdn=True)
    assert ring.vu.dtype == torch.bfloat16
    state0 = dev_f32(S0)
    ybf = bool(flags & _lib.RSSM_F_Y_BF16)
    y = torch.empty(sh.batch, T, sh.nheads, d, dtype=torch.bfloat16 if ybf else torch.float32, device="cuda")
    ytol = GDN_TOL + (2.0**-8 if ybf else 0.0)
    reqs = [o_gdn.GDNReplayRequest(S0[b].astype(np.float64), L, G, u_bf16=True) for b in range(sh.batch)]
    for r in range(R):
        st = synth.gdn_round_inputs(sh, seed, 4, r)
        s64 = gdn_step_f64(st)
        head_before = ring.head.cpu().numpy().copy()
        count_before = ring.count.cpu().numpy().copy()
        rd.gdn_replay_verify_T(dims, T, state0, ring, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                               dev_f32(st["g"]), dev_f32(st["beta"]), y)
        yh = _y_f64(y)
        ring_u = ring.entries().float().cpu().numpy()
        for b in range(sh.batch):
            yb, ub, fb = reqs[b].verify_round(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b], s64["beta"][b])
            assert rel_err(yh[b], yb) <= ytol, (r, b)
            slots = [(head_before[b] + count_before[b] + s) % L for s in range(T)]
            got_u = ring_u[b][:, slots].transpose(1, 0, 2)
            assert rel_err(got_u, o_gdn.round_bf16(ub)) <= U_TOL, (r, b)
            if fb:
                assert rel_err(state0[b].cpu().numpy(), reqs[b].S0) <= GDN_TOL, (r, b)
            reqs[b].commit(int(acc[r, b]))
        rd.replay_rollback(dims, ring, dev_i32(acc[r]))
    assert int(ring.err.item()) == 0
    rd.gdn_replay_flush(dims, state0, ring)
    for b in range(sh.batch):
        reqs[b].flush()
        assert rel_err(state0[b].cpu().numpy(), reqs[b].S0) <= GDN_TOL, b


def test_gdn_append_bf16_ring():
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=3, ngroups=32, capacity=8, T=1)
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    seed, steps = base.cfg_seed, 2 * L + 3
    S0 = synth.state0(sh, seed, 4)
    dims = rd.Dims(B, H, D, N, G, L, flags=_lib.RSSM_F_U_BF16 | _lib.RSSM_F_Y_BF16)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    y = torch.empty(B, H, D, dtype=torch.bfloat16, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    reqs = [o_gdn.GDNReplayRequest(S0[b].astype(np.float64), L, G, u_bf16=True) for b in range(B)]
    for t in range(steps):
        st = synth.gdn_round_inputs(sh, seed, 4, t)
        sq = {k_: np.ascontiguousarray(v_[:, 0]) for k_, v_ in st.items()}
        s64 = gdn_step_f64(sq)
        rd.gdn_replay_append_decode(dims, state0, ring, dev_bf16(sq["v"]), dev_bf16(sq["k"]), dev_bf16(sq["q"]),
                                    dev_f32(sq["g"]), dev_f32(sq["beta"]), y, flushed)
        yh = _y_f64(y)
        for b in range(B):
            yb, fb = reqs[b].decode_step(s64["v"][b], s64["k"][b], s64["q"][b], s64["g"][b], s64["beta"][b])
            assert rel_err(yh[b], yb) <= GDN_TOL + 2.0**-8, (t, b)
            assert bool(flushed[b].item()) == fb
            if fb:
                assert rel_err(state0[b].cpu().numpy(), reqs[b].S0) <= GDN_TOL, (t, b)
    assert int(ring.err.item()) == 0


def test_fused_front_end_bf16_y():
    """The fused front-end with bf16 outputs: y within 1e-3 + 2^-8 of the oracle's
    conv -> bf16 -> recurrence; the conv state still bit-exact; the checkpoint at
    every flush within the fp32 bar (the outputs' precision does not reach it)."""
    from oracle import conv1d as o_conv
    base = synth.WORKLOADS[0]
    d, G, L = 64, 2, 8
    sh = base.shape.with_(head_dim=d, ngroups=G, capacity=L)
    B, H, N = sh.batch, sh.nheads, sh.state_dim
    C = H * d + 2 * G * N
    seed, steps = base.cfg_seed, 2 * L + 3
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = synth.state0(sh, seed, 0)
    cs_bits, w_bits = synth.conv_layer(B, C, 4, seed, 0)
    dims = rd.Dims(B, H, d, N, G, L, flags=_lib.RSSM_F_Y_BF16)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    cs = [dev_bf16(cs_bits), dev_bf16(cs_bits)]
    w = dev_bf16(w_bits)
    y = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
    S = S0.astype(np.float64)
    cs64, W64 = synth.bf16_bits_to_f64(cs_bits), synth.bf16_bits_to_f64(w_bits)
    for t in range(steps):
        x_bits = synth.conv_step_input(B, C, seed, 0, t)
        dt = synth.mamba2_step_inputs(sh, seed, 0, t)["dt"]
        cin, cout = cs[t % 2], cs[(t + 1) % 2]
        rd.replay_append_decode_conv(dims, state0, ring, cin, cout, dev_bf16(x_bits), w, dev_f32(dt),
                                     dev_f32(dt_bias), dev_f32(A), y)
        out, cs64 = o_conv.update(cs64, synth.bf16_bits_to_f64(x_bits), W64)
        v, k, q = o_conv.split_xbc(o_conv.round_bf16(out), H, d, G, N)
        delta, a = o_m2.step_size_and_decay(dt.astype(np.float64), dt_bias.astype(np.float64),
                                            A.astype(np.float64))
        S, y_ref = o_m2.standard_step(S, v, k, q, delta, a, G)
        assert rel_err(_y_f64(y), y_ref) <= Y_TOL_BF16, t
        got = synth.bf16_bits_to_f64(cout.view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.array_equal(got, cs64), t
        if (t + 1) % L == 0:
            assert rel_err(state0.cpu().numpy(), S) <= S_TOL, t
    assert int(ring.err.item()) == 0


def test_commit_verify_bf16_y():
    """One launch per round with bf16 outputs (Mamba-2, T = 4): every draft's y
    within 1e-3 + 2^-8, the committed state after the final commit and flush
    within the fp32 bar."""
    from oracle import replay as o_rep
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=5, capacity=16, T=4)
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    seed, R = base.cfg_seed, 14
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, B, T)
    dims = rd.Dims(B, H, D, N, G, L, flags=_lib.RSSM_F_Y_BF16)
    ring = rd.Ring(dims)
    state0 = dev_f32(S0)
    y = torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda")
    S = S0.astype(np.float64)
    prev = dev_i32(np.zeros(B, int))
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(B)]
    for r in range(R):
        st = synth.mamba2_step_inputs(sh, seed, 2, r)
        rd.replay_commit_verify_T(dims, T, state0, ring, prev, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                  dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y)
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), G, acc[r])
        assert rel_err(_y_f64(y), y_ref) <= Y_TOL_BF16, r
        prev = dev_i32(acc[r])
    rd.replay_rollback(dims, ring, prev)
    assert ring.count.cpu().tolist() == [scheds[b][R - 1][4] for b in range(B)]
    rd.replay_flush(dims, state0, ring)
    assert rel_err(state0.cpu().numpy(), S) <= S_TOL
    assert int(ring.err.item()) == 0
