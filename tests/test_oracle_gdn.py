"""Pins for oracle.gdn: brute force with explicit Householder matrices, special
cases, the u-form invariant (ReplaySSM leaves outputs unchanged), and the chunk-wise
lower-triangular solve against textbook routines."""
import numpy as np
import pytest
import scipy.linalg

from oracle import gdn, rounding
from tests.util import tiny_gdn


def _explicit_state(S0, seq, b, h, g_of_h, t):
    """S_t = S_0 prod_i alpha_i (I - beta_i k_i k_i^T)
             + sum_i beta_i v_i k_i^T prod_{j>i} alpha_j (I - beta_j k_j k_j^T),
    products taken left to right in time, with explicit n x n matrices."""
    n = S0.shape[-1]
    I = np.eye(n)

    def M(i):
        k = seq[i]["k"][b, g_of_h]
        return np.exp(seq[i]["g"][b, h]) * (I - seq[i]["beta"][b, h] * np.outer(k, k))

    P = I.copy()
    for i in range(t + 1):
        P = P @ M(i)
    S = S0[b, h] @ P
    for i in range(t + 1):
        Q = I.copy()
        for j in range(i + 1, t + 1):
            Q = Q @ M(j)
        S = S + seq[i]["beta"][b, h] * np.outer(seq[i]["v"][b, h], seq[i]["k"][b, g_of_h]) @ Q
    return S


@pytest.mark.parametrize("G", [1, 2])
def test_householder_brute_force(G):
    rng = np.random.default_rng(40 + G)
    B, H, d, n, steps = 2, 2, 3, 4, 6
    S0, seq = tiny_gdn(rng, B, H, d, n, G, steps)
    S = S0
    for t, st in enumerate(seq):
        S, y = gdn.householder_step(S, st["v"], st["k"], st["q"], st["g"], st["beta"], G)
        for b in range(B):
            for h in range(H):
                ref = _explicit_state(S0, seq, b, h, h // (H // G), t)
                assert np.allclose(S[b, h], ref, rtol=0, atol=1e-12)
                assert np.allclose(y[b, h], ref @ st["q"][b, h // (H // G)], rtol=0, atol=1e-12)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    S0, seq = tiny_gdn(rng, 2, 3, 4, 5, 3, 5)
    S = S0
    decay = np.ones((2, 3))
    for st in seq:
        st["beta"] = np.zeros_like(st["beta"])
        S, _ = gdn.householder_step(S, st["v"], st["k"], st["q"], st["g"], st["beta"], 3)
        decay = decay * np.exp(st["g"])
    assert np.allclose(S, decay[:, :, None, None] * S0, rtol=1e-14, atol=0)


def test_delta_rule_write_property():
    """g = 0, beta = 1 and a unit key: the new state maps k_t to v_t exactly."""
    rng = np.random.default_rng(4)
    S0, seq = tiny_gdn(rng, 2, 2, 5, 7, 2, 4)
    S = S0
    for st in seq:
        st["g"] = np.zeros_like(st["g"])
        st["beta"] = np.ones_like(st["beta"])
        S, _ = gdn.householder_step(S, st["v"], st["k"], st["q"], st["g"], st["beta"], 2)
        Sk = np.einsum("bhdn,bhn->bhd", S, st["k"])
        assert np.allclose(Sk, st["v"], rtol=0, atol=1e-12)


def _drafts(rd):
    return rd


@pytest.mark.parametrize("L,T", [(8, 2), (16, 4), (6, 3)])
def test_gdn_replay_spec_equals_snapshot_semantics(L, T):
    """Caching u instead of the state leaves every output unchanged, through early
    flushes and rollbacks; the committed state after a final flush matches."""
    rng = np.random.default_rng(300 + L)
    B, H, d, n, G, R = 3, 2, 4, 5, 2, 25
    S0, rounds = tiny_gdn(rng, B, H, d, n, G, R, T=T)
    acc = rng.integers(0, T + 1, size=(R, B))
    reqs = [gdn.GDNReplayRequest(S0[b], L, G) for b in range(B)]
    S = S0
    nflush = 0
    for r, rd in enumerate(rounds):
        y_ref, S = gdn.spec_round_snapshot(S, rd, G, acc[r])
        for b in range(B):
            y, u, f = reqs[b].verify_round(rd["v"][b], rd["k"][b], rd["q"][b], rd["g"][b], rd["beta"][b])
            nflush += f
            assert np.allclose(y, y_ref[b], rtol=0, atol=1e-11), (r, b)
            reqs[b].commit(int(acc[r, b]))
    assert nflush > 0
    for b in range(B):
        reqs[b].flush()
        assert np.allclose(reqs[b].S0, S[b], rtol=0, atol=1e-11)


def test_gdn_replay_standard_decode_equals_recurrence():
    rng = np.random.default_rng(8)
    B, H, d, n, G, L, steps = 2, 2, 4, 6, 1, 5, 17
    S0, seq = tiny_gdn(rng, B, H, d, n, G, steps)
    reqs = [gdn.GDNReplayRequest(S0[b], L, G) for b in range(B)]
    S = S0
    for t, st in enumerate(seq):
        S, y_ref = gdn.householder_step(S, st["v"], st["k"], st["q"], st["g"], st["beta"], G)
        for b in range(B):
            y, f = reqs[b].decode_step(st["v"][b], st["k"][b], st["q"][b], st["g"][b], st["beta"][b])
            assert np.allclose(y, y_ref[b], rtol=0, atol=1e-12)
            assert f == ((t + 1) % L == 0)
            if f:
                assert np.allclose(reqs[b].S0, S[b], rtol=0, atol=1e-12)


def test_rebuilt_state_routes_agree():
    rng = np.random.default_rng(12)
    r = gdn.GDNReplayRequest(rng.standard_normal((3, 4, 5)), 8, 3)
    entries = [gdn._Entry(rng.standard_normal((3, 4)), rng.standard_normal((3, 5)),
                          rng.uniform(0.2, 1.0, 3)) for _ in range(6)]
    assert np.allclose(r.rebuilt_state(entries), r.rebuilt_state_closed(entries), rtol=0, atol=1e-13)


@pytest.mark.parametrize("T", [1, 2, 4, 6])
def test_chunkwise_solve_matches_serial_and_textbook(T):
    rng = np.random.default_rng(500 + T)
    d, n = 5, 7
    S_h = rng.standard_normal((d, n))
    v = rng.standard_normal((T, d))
    k = rng.standard_normal((T, n))
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((T, n)) / np.sqrt(n)
    g = -np.logaddexp(0.0, rng.standard_normal(T))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    U, Y, A, R = gdn.chunkwise_window(S_h, v, k, q, g, beta)
    # textbook triangular solve and a general dense solve of (I + A) U = R
    assert np.allclose(np.triu(A), 0.0)
    U_tri = scipy.linalg.solve_triangular(np.eye(T) + A, R, lower=True, unit_diagonal=True)
    U_gen = np.linalg.solve(np.eye(T) + A, R)
    assert np.allclose(U, U_tri, rtol=0, atol=1e-12)
    assert np.allclose(U, U_gen, rtol=0, atol=1e-12)
    # serial delta-rule window from S_h
    S = S_h
    for s in range(T):
        al = np.exp(g[s])
        u = beta[s] * (v[s] - al * (S @ k[s]))
        S = al * S + np.outer(u, k[s])
        assert np.allclose(U[s], u, rtol=0, atol=1e-12)
        assert np.allclose(Y[s], S @ q[s], rtol=0, atol=1e-12)


def test_bf16_corrections_follow_the_rounded_recurrence():
    """With the ring in bf16, a step's outputs use its correction unrounded and
    every later step sees the state built from rounded corrections:
        u_t = beta (v - alpha S k),  y_t = alpha S q + u_t (k . q),
        S <- alpha S + bf16(u_t) k^T,
    written out per head (the rounding itself is pinned in test_oracle_conv1d)."""
    rng = np.random.default_rng(12)
    B, H, d, n, G, L, steps = 2, 2, 4, 6, 1, 3, 11
    S0, seq = tiny_gdn(rng, B, H, d, n, G, steps)
    reqs = [gdn.GDNReplayRequest(S0[b], L, G, u_bf16=True) for b in range(B)]
    S = np.array(S0, dtype=np.float64)
    for t, st in enumerate(seq):
        for b in range(B):
            y, f = reqs[b].decode_step(st["v"][b], st["k"][b], st["q"][b], st["g"][b], st["beta"][b])
            for h in range(H):
                k, q = st["k"][b, 0], st["q"][b, 0]
                a = np.exp(st["g"][b, h])
                u = st["beta"][b, h] * (st["v"][b, h] - a * (S[b, h] @ k))
                assert np.allclose(y[h], a * (S[b, h] @ q) + u * (k @ q), rtol=0, atol=1e-12)
                S[b, h] = a * S[b, h] + np.outer(rounding.round_bf16(u), k)
            if f:
                assert np.allclose(reqs[b].S0, S[b], rtol=0, atol=1e-12)
    for b in range(B):
        for e in reqs[b].ring:
            if e is not None:
                assert np.array_equal(rounding.round_bf16(e.u), e.u)
