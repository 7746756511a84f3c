"""Pins for oracle.conv1d: stepping the state update equals a full causal
convolution of the input history (numpy.convolve) followed by SiLU, and the state
shift is exact."""
import numpy as np
import scipy.special

from oracle import conv1d


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
