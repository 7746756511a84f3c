"""The decode rounds captured once in a HIP graph and replayed (CUDA-Graph notes
of the method page: per-request flush decisions are read on the device at run
time, and commit/rollback is a device kernel, so one captured graph serves every
round with no host synchronisation inside it).

Each replay's inputs (drafts, accepted counts) are copied into the captured
buffers by eager work between replays, followed by a synchronisation; every
replay is checked against the oracle (y within 1e-3, pointers bit-exact, the
checkpoint within 1e-4 after a final flush)."""
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


def _copy_bf16(dst, bits):
    dst.copy_(dev_bf16(bits))


def test_verify_rollback_graph_replays():
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=6, nheads=8, ngroups=2, capacity=16, T=4)
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    seed, R = base.cfg_seed, 24
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, B, T)
    rounds = [synth.mamba2_step_inputs(sh, seed, 2, r) for r in range(R)]
    dims = rd.Dims(B, H, D, N, G, L)
    state0 = dev_f32(S0)
    sv, sk, sq = (torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda"),
                  torch.empty(B, T, G, N, dtype=torch.bfloat16, device="cuda"),
                  torch.empty(B, T, G, N, dtype=torch.bfloat16, device="cuda"))
    sdt = torch.empty(B, T, H, device="cuda")
    sacc = torch.zeros(B, dtype=torch.int32, device="cuda")
    y = torch.empty(B, T, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    Ab, biasb = dev_f32(A), dev_f32(dt_bias)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        ring_c, state_c = rd.Ring(dims), state0.clone()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            rd.replay_verify_T(dims, T, state_c, ring_c, sv, sk, sq, sdt, biasb, Ab, y, flushed)
            rd.replay_rollback(dims, ring_c, sacc)
    torch.cuda.synchronize()
    # capture records the launches without running them; start from a clean ring anyway
    for name in ("vu", "k", "meta", "err"):
        getattr(ring_c, name).zero_()
    state_c.copy_(state0)
    torch.cuda.synchronize()

    S = S0.astype(np.float64)
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(B)]
    for r in range(R):
        st = rounds[r]
        _copy_bf16(sv, st["v"])
        _copy_bf16(sk, st["k"])
        _copy_bf16(sq, st["q"])
        sdt.copy_(dev_f32(st["dt"]))
        sacc.copy_(dev_i32(acc[r]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), G, acc[r])
        e = rel_err(y.cpu().numpy(), y_ref)
        assert e <= Y_TOL, (r, e)
        fl = flushed.cpu().numpy()
        cnt = ring_c.count.cpu().numpy()
        for b in range(B):
            assert bool(fl[b]) == scheds[b][r][1], (r, b)
            assert cnt[b] == scheds[b][r][4], (r, b)
    assert int(ring_c.err.item()) == 0
    rd.replay_flush(dims, state_c, ring_c)
    assert rel_err(state_c.cpu().numpy(), S) <= S_TOL


def test_gdn_append_graph_replays():
    base = synth.WORKLOADS[4]
    sh = base.shape.with_(batch=3, nheads=8, ngroups=8, capacity=8, T=1)
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    seed, steps = base.cfg_seed, 2 * L + 3
    S0 = synth.state0(sh, seed, 4)
    dims = rd.Dims(B, H, D, N, G, L)
    ring = rd.Ring(dims, gdn=True)
    state0 = dev_f32(S0)
    sv = torch.empty(B, H, D, dtype=torch.bfloat16, device="cuda")
    sk = torch.empty(B, G, N, dtype=torch.bfloat16, device="cuda")
    sq = torch.empty(B, G, N, dtype=torch.bfloat16, device="cuda")
    sg, sb = torch.empty(B, H, device="cuda"), torch.empty(B, H, device="cuda")
    y = torch.empty(B, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    state_c = state0.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rd.gdn_replay_append_decode(dims, state_c, ring, sv, sk, sq, sg, sb, y, flushed)
    torch.cuda.synchronize()
    for name in ("vu", "k", "meta", "err"):
        getattr(ring, name).zero_()
    state_c.copy_(state0)
    torch.cuda.synchronize()
    S = S0.astype(np.float64)
    for t in range(steps):
        st = synth.gdn_round_inputs(sh, seed, 4, t)
        sq_ = {k_: np.ascontiguousarray(v_[:, 0]) for k_, v_ in st.items()}
        _copy_bf16(sv, sq_["v"])
        _copy_bf16(sk, sq_["k"])
        _copy_bf16(sq, sq_["q"])
        sg.copy_(dev_f32(sq_["g"]))
        sb.copy_(dev_f32(sq_["beta"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        s64 = gdn_step_f64(sq_)
        S, y_ref = o_gdn.householder_step(S, s64["v"], s64["k"], s64["q"], s64["g"], s64["beta"], G)
        assert rel_err(y.cpu().numpy(), y_ref) <= Y_TOL, t
        fl = (t + 1) % L == 0
        assert bool(torch.all(flushed == int(fl))), t
        if fl:
            assert rel_err(state_c.cpu().numpy(), S) <= S_TOL, t
    assert int(ring.err.item()) == 0


def test_commit_verify_graph_replays():
    """One launch per speculative round, captured once: each replay commits the
    previous round's accepted counts (copied into the captured buffer between
    replays) and verifies the next window; the last window is committed eagerly
    before the final flush."""
    base = synth.WORKLOADS[2]
    sh = base.shape.with_(batch=5, nheads=8, ngroups=2, capacity=16, T=4)
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    seed, R = base.cfg_seed, 20
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    acc = synth.accept_draws(seed, 2, R, B, T)
    rounds = [synth.mamba2_step_inputs(sh, seed, 2, r) for r in range(R)]
    dims = rd.Dims(B, H, D, N, G, L)
    state0 = dev_f32(S0)
    sv, sk, sq = (torch.empty(B, T, H, D, dtype=torch.bfloat16, device="cuda"),
                  torch.empty(B, T, G, N, dtype=torch.bfloat16, device="cuda"),
                  torch.empty(B, T, G, N, dtype=torch.bfloat16, device="cuda"))
    sdt = torch.empty(B, T, H, device="cuda")
    sacc = torch.zeros(B, dtype=torch.int32, device="cuda")
    y = torch.empty(B, T, H, D, device="cuda")
    flushed = torch.zeros(B, dtype=torch.int32, device="cuda")
    Ab, biasb = dev_f32(A), dev_f32(dt_bias)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        ring_c, state_c = rd.Ring(dims), state0.clone()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            rd.replay_commit_verify_T(dims, T, state_c, ring_c, sacc, sv, sk, sq, sdt, biasb, Ab, y, flushed)
    torch.cuda.synchronize()
    for name in ("vu", "k", "meta", "err"):
        getattr(ring_c, name).zero_()
    state_c.copy_(state0)
    torch.cuda.synchronize()

    S = S0.astype(np.float64)
    scheds = [o_rep.pointer_schedule_spec(L, T, acc[:, b]) for b in range(B)]
    for r in range(R):
        st = rounds[r]
        _copy_bf16(sv, st["v"])
        _copy_bf16(sk, st["k"])
        _copy_bf16(sq, st["q"])
        sdt.copy_(dev_f32(st["dt"]))
        sacc.copy_(dev_i32(acc[r - 1] if r > 0 else np.zeros(B, int)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                            A.astype(np.float64), G, acc[r])
        e = rel_err(y.cpu().numpy(), y_ref)
        assert e <= Y_TOL, (r, e)
        fl = flushed.cpu().numpy()
        hd, cnt, pd = (x.cpu().numpy() for x in ring_c.pointers())
        for b in range(B):
            assert bool(fl[b]) == scheds[b][r][1], (r, b)
            assert (hd[b], cnt[b], pd[b]) == (scheds[b][r][2], scheds[b][r][3], T), (r, b)
    rd.replay_rollback(dims, ring_c, dev_i32(acc[R - 1]))
    assert ring_c.count.cpu().tolist() == [scheds[b][R - 1][4] for b in range(B)]
    assert int(ring_c.err.item()) == 0
    rd.replay_flush(dims, state_c, ring_c)
    assert rel_err(state_c.cpu().numpy(), S) <= S_TOL
