"""Pins for oracle.mamba2: brute force of the unrolled history form, closed forms,
special cases that reduce to textbook routines."""
import math

import numpy as np
import pytest

from oracle import mamba2
from tests.util import tiny_mamba2


def _py_discretise(dt, bias, A):
    x = dt + bias
    delta = x if x > 20 else math.log1p(math.exp(x))
    return delta, math.exp(A * delta)


def _brute_force(S0, seq, dt_bias, A, G):
    """The unrolled form of the core-idea section, plus the decayed checkpoint:
    S_t = (prod_{i<=t} a_i) S_0 + sum_{i<=t} (prod_{i<j<=t} a_j) Delta_i v_i k_i^T,
    y_t = S_t q_t, with scalar Python loops and an independent discretisation."""
    B, H, d, n = S0.shape
    per = H // G
    ys = np.zeros((len(seq), B, H, d))
    Sfin = np.zeros_like(S0)
    for b in range(B):
        for h in range(H):
            g = h // per
            da = [_py_discretise(float(st["dt"][b, h]), float(dt_bias[h]), float(A[h])) for st in seq]
            for t in range(len(seq)):
                for r in range(d):
                    row = []
                    for c in range(n):
                        prod_all = 1.0
                        for i in range(t + 1):
                            prod_all *= da[i][1]
                        acc = prod_all * float(S0[b, h, r, c])
                        for i in range(t + 1):
                            w = 1.0
                            for j in range(i + 1, t + 1):
                                w *= da[j][1]
                            acc += w * da[i][0] * float(seq[i]["v"][b, h, r]) * float(seq[i]["k"][b, g, c])
                        row.append(acc)
                    ys[t, b, h, r] = sum(row[c] * float(seq[t]["q"][b, g, c]) for c in range(n))
                    if t == len(seq) - 1:
                        Sfin[b, h, r, :] = row
    return ys, Sfin


@pytest.mark.parametrize("d,n,G,steps", [(2, 3, 1, 12), (3, 4, 2, 7), (4, 2, 2, 9)])
def test_brute_force_unrolled(d, n, G, steps):
    rng = np.random.default_rng(1000 + d * 10 + n)
    S0, seq, dt_bias, A = tiny_mamba2(rng, 1, 2, d, n, G, steps)
    ys, Ss = mamba2.run_standard(S0, seq, dt_bias, A, G)
    ref_y, ref_S = _brute_force(S0, seq, dt_bias, A, G)
    assert np.max(np.abs(np.stack(ys) - ref_y)) <= 1e-12 * max(1.0, np.max(np.abs(ref_y)))
    assert np.max(np.abs(Ss[-1] - ref_S)) <= 1e-12 * max(1.0, np.max(np.abs(ref_S)))


def test_geometric_series_closed_form():
    """d = n = 1 with constant inputs: S_t = a^t S_0 + Delta v k (1 - a^t) / (1 - a)."""
    S0 = np.array([[[[0.7]]]])
    A = np.array([-1.3])
    bias = np.array([0.2])
    dt, v, k, q = 0.4, 1.5, -0.8, 2.0
    delta = math.log1p(math.exp(dt + 0.2))
    a = math.exp(-1.3 * delta)
    seq = [{"v": np.full((1, 1, 1), v), "k": np.full((1, 1, 1), k), "q": np.full((1, 1, 1), q),
            "dt": np.full((1, 1), dt)} for _ in range(25)]
    ys, Ss = mamba2.run_standard(S0, seq, bias, A, 1)
    for t in range(1, 26):
        S_t = a ** t * 0.7 + delta * v * k * (1 - a ** t) / (1 - a)
        assert abs(Ss[t - 1][0, 0, 0, 0] - S_t) <= 1e-13
        assert abs(ys[t - 1][0, 0, 0] - S_t * q) <= 1e-13


def test_zero_decay_is_causal_linear_attention():
    """A = 0 gives a = 1: y_t = S_0 q_t + sum_{j<=t} Delta_j (k_j . q_t) v_j, i.e.
    Y = Q S_0^T + (tril(Q K^T) * Delta) V, one masked matmul per head."""
    rng = np.random.default_rng(7)
    B, H, d, n, G, T = 2, 4, 5, 6, 2, 11
    S0, seq, dt_bias, _ = tiny_mamba2(rng, B, H, d, n, G, T)
    A = np.zeros(H)
    ys, _ = mamba2.run_standard(S0, seq, dt_bias, A, G)
    Y = np.stack(ys)                                   # [T,B,H,d]
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            Q = np.stack([st["q"][b, g] for st in seq])      # [T,n]
            K = np.stack([st["k"][b, g] for st in seq])
            V = np.stack([st["v"][b, h] for st in seq])      # [T,d]
            Dl = np.log1p(np.exp(np.array([st["dt"][b, h] for st in seq]) + dt_bias[h]))
            ref = Q @ S0[b, h].T + (np.tril(Q @ K.T) * Dl[None, :]) @ V
            assert np.allclose(Y[:, b, h], ref, rtol=0, atol=1e-12)


def test_zero_state_single_step_inner_product():
    """Zero initial state, one step: y = Delta (v k^T) q = Delta v (k^T q)."""
    rng = np.random.default_rng(3)
    S0, seq, dt_bias, A = tiny_mamba2(rng, 3, 4, 8, 16, 4, 1, s0_scale=0.0)
    ys, _ = mamba2.run_standard(S0, seq, dt_bias, A, 4)
    st = seq[0]
    delta = np.log1p(np.exp(st["dt"] + dt_bias))
    ref = delta[:, :, None] * st["v"] * np.sum(st["k"] * st["q"], axis=-1)[:, :, None]
    assert np.allclose(ys[0], ref, rtol=0, atol=1e-14)


def test_softplus_pins():
    x = np.linspace(-30, 30, 601)
    assert np.allclose(mamba2.softplus(x), np.logaddexp(0.0, x), rtol=1e-15, atol=1e-300)
    assert mamba2.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-16)
    assert np.allclose(mamba2.softplus(x) - mamba2.softplus(-x), x, atol=1e-12)


def test_group_sharing_matches_repeated_keys():
    """G groups of k/q equal H groups where each head gets its group's k/q."""
    rng = np.random.default_rng(11)
    B, H, d, n, G = 2, 6, 3, 4, 2
    S0, seq, dt_bias, A = tiny_mamba2(rng, B, H, d, n, G, 5)
    ys_g, Ss_g = mamba2.run_standard(S0, seq, dt_bias, A, G)
    rep = [dict(st, k=np.repeat(st["k"], H // G, axis=1), q=np.repeat(st["q"], H // G, axis=1))
           for st in seq]
    ys_h, Ss_h = mamba2.run_standard(S0, rep, dt_bias, A, H)
    assert np.array_equal(np.stack(ys_g), np.stack(ys_h))
    assert np.array_equal(Ss_g[-1], Ss_h[-1])


def test_spec_snapshot_full_accept_is_plain_decode():
    """Accepting every draft of every round equals plain decode of all drafts in order;
    accepting none leaves the committed state untouched."""
    rng = np.random.default_rng(5)
    B, H, d, n, G, T, R = 2, 2, 3, 4, 1, 3, 4
    S0, rounds, dt_bias, A = tiny_mamba2(rng, B, H, d, n, G, R, T=T)
    flat = [{key: rd[key][:, s] for key in rd} for rd in rounds for s in range(T)]
    ys_plain, Ss_plain = mamba2.run_standard(S0, flat, dt_bias, A, G)
    S = S0
    for r, rd in enumerate(rounds):
        y, S = mamba2.spec_round_snapshot(S, rd, dt_bias, A, G, np.full(B, T))
        for s in range(T):
            assert np.allclose(y[:, s], ys_plain[r * T + s], rtol=0, atol=1e-13)
    assert np.allclose(S, Ss_plain[-1], rtol=0, atol=1e-13)
    y0, S_none = mamba2.spec_round_snapshot(S0, rounds[0], dt_bias, A, G, np.zeros(B, int))
    assert np.array_equal(S_none, S0)
