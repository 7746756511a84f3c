"""Pins for oracle.replay: the page's invariant that ReplaySSM leaves the outputs of
the standard recurrence unchanged (plain decode, after flushes, after speculative
rollback), the flush schedules, and the ring-pointer rules."""
import numpy as np
import pytest

from oracle import mamba2, replay
from ssm_recurrent_decode_amd import synth
from tests.util import tiny_mamba2


def _check_replay_matches_standard(S0, seq, dt_bias, A, L, G, tol=1e-10):
    ys_std, Ss_std = mamba2.run_standard(S0, seq, dt_bias, A, G)
    ys_rep, flags, reqs = replay.run_standard(S0, seq, dt_bias, A, L, G)
    scale = max(1.0, max(np.max(np.abs(y)) for y in ys_std))
    for t in range(len(seq)):
        assert np.max(np.abs(ys_rep[t] - ys_std[t])) <= tol * scale, t
    # S_0 equals the standard state right after every flush
    B = S0.shape[0]
    S0_track = [np.array(S0[b]) for b in range(B)]
    reqs2 = [replay.ReplayRequest(S0[b], L, G) for b in range(B)]
    for t, st in enumerate(seq):
        delta, a = mamba2.step_size_and_decay(st["dt"], dt_bias, A)
        for b in range(B):
            _, f = reqs2[b].decode_step(st["v"][b], st["k"][b], st["q"][b], delta[b], a[b])
            if f:
                assert np.max(np.abs(reqs2[b].S0 - Ss_std[t][b])) <= tol * max(1.0, np.max(np.abs(Ss_std[t][b])))
    return flags


@pytest.mark.parametrize("L,G,steps", [(4, 1, 13), (3, 2, 10), (8, 2, 25)])
def test_replay_equals_standard_tiny(L, G, steps):
    rng = np.random.default_rng(100 + L)
    S0, seq, dt_bias, A = tiny_mamba2(rng, 3, 4, 5, 6, G, steps)
    flags = _check_replay_matches_standard(S0, seq, dt_bias, A, L, G)
    # flush exactly on the steps whose append fills the ring (1-based t = L, 2L, ...)
    for t, f in enumerate(flags):
        assert bool(np.all(f)) == ((t + 1) % L == 0) and bool(np.all(f)) == bool(np.any(f))


def test_replay_ring_dominant_variant():
    """S_0 = 0, dt_bias = 0, A in [-1, -0.1]: the ring terms carry the output, so a
    wrong decay exponent or an off-by-one in s_j would show at any tolerance."""
    rng = np.random.default_rng(21)
    H = 4
    A = -rng.uniform(0.1, 1.0, H)
    S0, seq, dt_bias, _ = tiny_mamba2(rng, 2, H, 6, 8, 2, 30, s0_scale=0.0,
                                      dt_bias=np.zeros(H), A=A)
    _check_replay_matches_standard(S0, seq, dt_bias, A, 8, 2)


def test_replay_equals_standard_config0_full():
    """The tiny Mamba-2 workload in full: B=4, H=8, d=64, n=128, G=1, L=8, 32 steps
    with bf16 inputs.  Four flushes, at steps 8, 16, 24, 32."""
    wl = synth.WORKLOADS[0]
    sh, seed = wl.shape, wl.cfg_seed
    A, dt_bias = synth.mamba2_head_params(sh, seed, 0)
    S0 = synth.state0(sh, seed, 0).astype(np.float64)
    seq = []
    for t in range(wl.steps):
        st = synth.mamba2_step_inputs(sh, seed, 0, t)
        seq.append({"v": synth.bf16_bits_to_f64(st["v"]), "k": synth.bf16_bits_to_f64(st["k"]),
                    "q": synth.bf16_bits_to_f64(st["q"]), "dt": st["dt"].astype(np.float64)})
    flags = _check_replay_matches_standard(S0, seq, dt_bias.astype(np.float64),
                                           A.astype(np.float64), sh.capacity, sh.ngroups)
    flush_steps = [t + 1 for t, f in enumerate(flags) if f.all()]
    assert flush_steps == [8, 16, 24, 32]


def test_explicit_flush_then_continue():
    rng = np.random.default_rng(33)
    B, H, d, n, G, L = 2, 2, 3, 5, 1, 6
    S0, seq, dt_bias, A = tiny_mamba2(rng, B, H, d, n, G, 17)
    ys_std, Ss_std = mamba2.run_standard(S0, seq, dt_bias, A, G)
    reqs = [replay.ReplayRequest(S0[b], L, G) for b in range(B)]
    for t, st in enumerate(seq):
        delta, a = mamba2.step_size_and_decay(st["dt"], dt_bias, A)
        for b in range(B):
            y, _ = reqs[b].decode_step(st["v"][b], st["k"][b], st["q"][b], delta[b], a[b])
            assert np.allclose(y, ys_std[t][b], rtol=0, atol=1e-12)
            if t in (2, 9, 10):
                reqs[b].flush()
                assert reqs[b].count == 0
                assert np.allclose(reqs[b].S0, Ss_std[t][b], rtol=0, atol=1e-12)


def _spec_check(B, H, d, n, G, L, T, R, seed, s0_scale=1.0):
    rng = np.random.default_rng(seed)
    S0, rounds, dt_bias, A = tiny_mamba2(rng, B, H, d, n, G, R, T=T, s0_scale=s0_scale)
    acc = rng.integers(0, T + 1, size=(R, B))
    ys, flags, starts, reqs = replay.run_spec(S0, rounds, dt_bias, A, L, G, acc)
    S = S0
    for r, rd in enumerate(rounds):
        y_ref, S = mamba2.spec_round_snapshot(S, rd, dt_bias, A, G, acc[r])
        assert np.max(np.abs(ys[r] - y_ref)) <= 1e-10 * max(1.0, np.max(np.abs(y_ref))), r
    for b in range(B):
        reqs[b].flush()
        assert np.max(np.abs(reqs[b].S0 - S[b])) <= 1e-10 * max(1.0, np.max(np.abs(S[b])))
    return np.stack(flags), np.stack(starts), acc


@pytest.mark.parametrize("L,T", [(8, 2), (8, 4), (16, 4), (9, 3)])
def test_spec_replay_equals_snapshot_semantics(L, T):
    """y of every draft position (rejected ones included) and the committed state
    equal the per-draft snapshot semantics, whatever is accepted."""
    flags, starts, acc = _spec_check(3, 4, 5, 6, 2, L, T, 30, seed=200 + L + T)
    assert flags.any(), "the run should cross at least one early flush"


def test_spec_window_never_truncated_and_flush_as_late_as_possible():
    """The early flush keeps room for a whole window at every round start
    (count + T <= L) and fires only when accepting all T drafts would otherwise
    leave less than a window free for the next round."""
    L, T, R = 16, 4, 200
    flags, starts, acc = _spec_check(4, 2, 2, 3, 1, L, T, R, seed=77)
    B = starts.shape[1]
    for r in range(R):
        for b in range(B):
            c = int(starts[r, b])
            assert c + T <= L
            worst_next = c + T          # count before the next round if all T are accepted
            assert bool(flags[r, b]) == (worst_next + T > L)
            nxt = (0 if flags[r, b] else c) + int(acc[r, b])
            if r + 1 < R:
                assert starts[r + 1, b] == nxt


def test_spec_config0_shape_with_rollbacks():
    """Config-0 sizes (d=64, n=128) with T=4, L=16 and random acceptance."""
    _spec_check(2, 8, 64, 128, 1, 16, 4, 12, seed=9, s0_scale=np.sqrt(0.1))


def test_integer_schedules_match_full_oracle():
    rng = np.random.default_rng(55)
    L, T, R = 16, 4, 60
    S0, rounds, dt_bias, A = tiny_mamba2(rng, 1, 1, 2, 3, 1, R, T=T)
    acc = rng.integers(0, T + 1, size=R)
    r = replay.ReplayRequest(S0[0], L, 1)
    sched = replay.pointer_schedule_spec(L, T, acc)
    for i, rd in enumerate(rounds):
        delta, a = mamba2.step_size_and_decay(rd["dt"], dt_bias, A)
        c0 = r.count
        _, f = r.verify_round(rd["v"][0], rd["k"][0], rd["q"][0], delta[0], a[0])
        assert sched[i][:4] == (c0, f, r.head, r.count)
        r.commit(int(acc[i]))
        assert sched[i][4] == r.count
    S0, seq, dt_bias, A = tiny_mamba2(rng, 1, 1, 2, 3, 1, 40)
    r = replay.ReplayRequest(S0[0], 8, 1)
    sched = replay.pointer_schedule_standard(8, 40)
    for t, st in enumerate(seq):
        delta, a = mamba2.step_size_and_decay(st["dt"], dt_bias, A)
        _, f = r.decode_step(st["v"][0], st["k"][0], st["q"][0], delta[0], a[0])
        assert sched[t] == (r.head, r.count, f)
