"""Plant plausible mistakes in the oracle (on the CPU only) and check that one of the
pins catches each: a dropped term, a wrong sign, an off-by-one, a transposed or
swapped operand, a wrong group mapping."""
import numpy as np
import pytest

from oracle import conv1d, gdn, mamba2, replay, rounding
from tests import test_oracle_conv1d as t_conv
from tests import test_oracle_gdn as t_gdn
from tests import test_oracle_mamba2 as t_m2
from tests import test_oracle_replay as t_rep


def _fails(fn, *a, **kw):
    with pytest.raises(AssertionError):
        fn(*a, **kw)


def test_dropped_step_size_is_caught(monkeypatch):
    orig = mamba2.standard_step
    monkeypatch.setattr(mamba2, "standard_step",
                        lambda S, v, k, q, delta, a, G: orig(S, v, k, q, np.ones_like(delta), a, G))
    _fails(t_m2.test_brute_force_unrolled, 2, 3, 1, 12)


def test_wrong_decay_sign_is_caught(monkeypatch):
    def bad(dt, dt_bias, A):
        delta = mamba2.softplus(np.asarray(dt) + dt_bias)
        return delta, np.exp(-np.asarray(A) * delta)
    monkeypatch.setattr(mamba2, "step_size_and_decay", bad)
    _fails(t_m2.test_brute_force_unrolled, 3, 4, 2, 7)


def test_missing_bias_is_caught(monkeypatch):
    def bad(dt, dt_bias, A):
        delta = mamba2.softplus(np.asarray(dt))
        return delta, np.exp(np.asarray(A) * delta)
    monkeypatch.setattr(mamba2, "step_size_and_decay", bad)
    _fails(t_m2.test_brute_force_unrolled, 4, 2, 2, 9)


def test_wrong_group_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(mamba2, "group_of_head", lambda H, G: np.arange(H) % G)
    _fails(t_m2.test_group_sharing_matches_repeated_keys)


def test_off_by_one_decay_weight_is_caught(monkeypatch):
    def bad(entries, H):
        abar = np.ones(H)
        for e in entries:
            abar = abar * e.a
        s = []
        for j in range(len(entries)):
            w = np.array(entries[j].delta, dtype=np.float64)
            for i in range(j, len(entries)):          # includes a_j itself
                w = w * entries[i].a
            s.append(w)
        return abar, s
    monkeypatch.setattr(replay.ReplayRequest, "_weights", staticmethod(bad))
    _fails(t_rep.test_replay_equals_standard_tiny, 4, 1, 13)


def test_checkpoint_decay_dropped_is_caught(monkeypatch):
    orig = replay.ReplayRequest._weights

    def bad(entries, H):
        abar, s = orig(entries, H)
        return np.ones_like(abar), s
    monkeypatch.setattr(replay.ReplayRequest, "_weights", staticmethod(bad))
    _fails(t_rep.test_replay_equals_standard_tiny, 3, 2, 10)


def test_draft_reads_wrong_prefix_is_caught(monkeypatch):
    def bad_verify(self, v, k, q, delta, a):
        T = v.shape[0]
        c = self.count
        for s in range(T):
            self.ring[(self.head + c + s) % self.L] = replay._Entry(v[s], k[s], delta[s], a[s])
        self.pending = T
        ys = [self._read(q[s], self._logical(c + s)) for s in range(T)]   # misses its own draft
        flushed = False
        if c + 2 * T > self.L:
            if c > 0:
                self._fold(self._logical(c))
            self.head = (self.head + c) % self.L
            self.count = 0
            flushed = True
        return np.stack(ys), flushed
    monkeypatch.setattr(replay.ReplayRequest, "verify_round", bad_verify)
    _fails(t_rep.test_spec_replay_equals_snapshot_semantics, 8, 2)


def test_commit_off_by_one_is_caught(monkeypatch):
    def bad_commit(self, accepted):
        self.count += max(accepted - 1, 0)
        self.pending = 0
    monkeypatch.setattr(replay.ReplayRequest, "commit", bad_commit)
    _fails(t_rep.test_spec_replay_equals_snapshot_semantics, 16, 4)


def test_late_flush_rule_is_caught(monkeypatch):
    """Flushing only when h + T > L (instead of h + 2T > L) lets the window be
    truncated after a round that accepts every draft."""
    def bad(self, v, k, q, delta, a):
        T = v.shape[0]
        c = self.count
        assert self.pending == 0 and c + T <= self.L, "window would be truncated"
        for s in range(T):
            self.ring[(self.head + c + s) % self.L] = replay._Entry(v[s], k[s], delta[s], a[s])
        self.pending = T
        ys = [self._read(q[s], self._logical(c + s + 1)) for s in range(T)]
        flushed = False
        if c + T > self.L:
            self._fold(self._logical(c))
            self.head = (self.head + c) % self.L
            self.count = 0
            flushed = True
        return np.stack(ys), flushed
    monkeypatch.setattr(replay.ReplayRequest, "verify_round", bad)
    _fails(t_rep.test_spec_window_never_truncated_and_flush_as_late_as_possible)


def test_gdn_erase_with_wrong_vector_is_caught(monkeypatch):
    orig = gdn.householder_step
    monkeypatch.setattr(gdn, "householder_step",
                        lambda S, v, k, q, g, beta, G: orig(S, v, q, q, g, beta, G))
    _fails(t_gdn.test_householder_brute_force, 1)


def test_gdn_transposed_outer_product_is_caught(monkeypatch):
    def bad(S, v, k, q, g, beta, G):
        S = np.asarray(S, np.float64)
        B, H, d, n = S.shape
        grp = mamba2.group_of_head(H, G)
        kh, qh = k[:, grp, :], q[:, grp, :]
        alpha = np.exp(g)
        Sk = np.sum(S * kh[:, :, None, :], axis=-1)
        erased = S - beta[:, :, None, None] * (Sk[:, :, :, None] * kh[:, :, None, :])
        # k v^T instead of v k^T (shapes agree only because d == n below)
        S_new = alpha[:, :, None, None] * erased + beta[:, :, None, None] * (
            kh[:, :, :, None] * v[:, :, None, :])
        y = np.sum(S_new * qh[:, :, None, :], axis=-1)
        return S_new, y
    monkeypatch.setattr(gdn, "householder_step", bad)
    rng = np.random.default_rng(0)
    # square state so the transposed operand has a valid shape
    from tests.util import tiny_gdn
    S0, seq = tiny_gdn(rng, 1, 1, 3, 3, 1, 2)
    S, _ = gdn.householder_step(S0, seq[0]["v"], seq[0]["k"], seq[0]["q"], seq[0]["g"], seq[0]["beta"], 1)
    ref = t_gdn._explicit_state(S0, seq, 0, 0, 0, 0)
    assert not np.allclose(S[0, 0], ref, atol=1e-9)


def test_gdn_substitution_sign_is_caught(monkeypatch):
    orig = gdn.chunkwise_window

    def bad(S_h, v, k, q, g, beta):
        U, Y, A, R = orig(S_h, v, k, q, g, beta)
        T = len(g)
        U2 = np.zeros_like(U)
        for s in range(T):
            acc = np.array(R[s])
            for sp in range(s):
                acc = acc + A[s, sp] * U2[sp]          # sign flipped
            U2[s] = acc
        return U2, Y, A, R
    monkeypatch.setattr(gdn, "chunkwise_window", bad)
    _fails(t_gdn.test_chunkwise_solve_matches_serial_and_textbook, 4)


def test_gdn_gate_dropped_from_correction_is_caught(monkeypatch):
    orig = gdn.GDNReplayRequest.verify_round

    def bad(self, v, k, q, g, beta):
        return orig(self, v, k, q, np.zeros_like(g), beta)
    monkeypatch.setattr(gdn.GDNReplayRequest, "verify_round", bad)
    _fails(t_gdn.test_gdn_replay_spec_equals_snapshot_semantics, 8, 2)


def test_conv_reversed_taps_are_caught(monkeypatch):
    orig = conv1d.update
    monkeypatch.setattr(conv1d, "update", lambda s, x, w: orig(s, x, w[:, ::-1]))
    _fails(t_conv.test_conv_update_equals_full_causal_convolution)


def test_bf16_rounding_ties_away_is_caught(monkeypatch):
    def bad(x):
        x = np.asarray(x, np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(m * 256.0 + np.copysign(0.5, m)), e - 8)   # halves away from zero
    monkeypatch.setattr(rounding, "round_bf16", bad)
    _fails(t_conv.test_round_bf16_ties_and_carry)


def test_swapped_key_and_query_channels_are_caught(monkeypatch):
    def bad(out, H, d, G, n):
        Bt = out.shape[0]
        v = out[:, :H * d].reshape(Bt, H, d)
        q = out[:, H * d:H * d + G * n].reshape(Bt, G, n)
        k = out[:, H * d + G * n:].reshape(Bt, G, n)
        return v, k, q
    monkeypatch.setattr(conv1d, "split_xbc", bad)
    _fails(t_conv.test_split_xbc_channel_order)


def test_bf16_correction_rounded_for_its_own_output_is_caught(monkeypatch):
    orig_decode = gdn.GDNReplayRequest.decode_step

    def bad(self, v, k, q, g, beta):
        # outputs computed as if the step's own correction were already rounded
        S_h = self.rebuilt_state_closed(self._logical(self.count))
        alpha = np.exp(g)
        kh, qh = k[self.grp], q[self.grp]
        u = beta[:, None] * (v - alpha[:, None] * np.sum(S_h * kh[:, None, :], axis=-1))
        y_bad = alpha[:, None] * np.sum(S_h * qh[:, None, :], axis=-1) + \
            self._cached(u) * np.sum(kh * qh, axis=-1)[:, None]
        _, flushed = orig_decode(self, v, k, q, g, beta)
        return y_bad, flushed
    monkeypatch.setattr(gdn.GDNReplayRequest, "decode_step", bad)
    _fails(t_gdn.test_bf16_corrections_follow_the_rounded_recurrence)
