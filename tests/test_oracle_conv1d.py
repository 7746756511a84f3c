"""Pins for oracle.conv1d: stepping the state update equals a full causal
convolution of the input history (numpy.convolve) followed by SiLU, and the state
shift is exact."""
import numpy as np
import scipy.special

from oracle import conv1d, rounding


def test_conv_update_equals_full_causal_convolution():
    rng = np.random.default_rng(1)
    B, C, W, steps = 3, 5, 4, 9
    state = rng.standard_normal((B, C, W - 1))
    weight = rng.standard_normal((C, W))
    xs = rng.standard_normal((steps, B, C))
    outs = []
    st = state
    for t in range(steps):
        o, st = conv1d.update(st, xs[t], weight)
        outs.append(o)
    for b in range(B):
        for c in range(C):
            hist = np.concatenate([state[b, c], xs[:, b, c]])     # x_{-3..-1}, x_0..x_{steps-1}
            full = np.convolve(hist, weight[c][::-1])            # tap W-1 multiplies the newest input
            pre = full[W - 1: W - 1 + steps]
            ref = pre * scipy.special.expit(pre)
            got = np.array([outs[t][b, c] for t in range(steps)])
            assert np.allclose(got, ref, rtol=1e-14, atol=1e-14)
            assert np.array_equal(st[b, c], hist[-(W - 1):])


def test_silu_special_values():
    assert conv1d.silu(np.float64(0.0)) == 0.0
    x = np.array([40.0, -40.0, 1.0])
    got = conv1d.silu(x)
    assert abs(got[0] - 40.0) < 1e-12 and abs(got[1]) < 1e-15
    assert abs(got[2] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16


def test_round_bf16_ties_and_carry():
    one = 1.0
    assert rounding.round_bf16(one + 2.0**-8) == one                   # tie -> even (1.0)
    assert rounding.round_bf16(one + 3 * 2.0**-8) == one + 2.0**-6     # tie -> even mantissa
    assert rounding.round_bf16(one + 2.0**-8 + 2.0**-20) == one + 2.0**-7
    assert rounding.round_bf16(2.0 - 2.0**-9) == 2.0                   # carry into the exponent
    assert rounding.round_bf16(-(one + 2.0**-7)) == -(one + 2.0**-7)   # representable stays
    assert rounding.round_bf16(0.0) == 0.0


def test_round_bf16_matches_library_conversion():
    torch = __import__("pytest").importorskip("torch")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = rounding.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # within half an ulp (at most 2^-8 of |x|: 8 significand bits) and idempotent
    assert np.all(np.abs(got - x) <= np.abs(x) * 2.0**-8)
    assert np.array_equal(rounding.round_bf16(got), got)


def test_split_xbc_channel_order():
    H, d, G, n = 2, 3, 1, 4
    out = np.arange(2 * (H * d + 2 * G * n), dtype=np.float64).reshape(2, -1)
    v, k, q = conv1d.split_xbc(out, H, d, G, n)
    assert v[1, 1, 2] == out[1, 1 * d + 2]
    assert k[0, 0, 3] == out[0, H * d + 3]
    assert q[1, 0, 0] == out[1, H * d + G * n]
