"""The input generators: bf16 rounding against torch's CPU conversion, the stated
distributions, and independence of the keyed streams."""
import numpy as np
import torch

from ssm_recurrent_decode_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -1e-38, 1.00390625, 1.01171875], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_distributions_and_shapes():
    sh = synth.WORKLOADS[1].shape
    A, bias = synth.mamba2_head_params(sh, 1, 1)
    assert A.shape == (32,) and np.all(A <= -1.0) and np.all(A >= -16.0)
    assert np.all(bias >= -4.0) and np.all(bias <= -2.0)
    st = synth.mamba2_step_inputs(sh, 1, 1, 0)
    assert st["v"].shape == (256, 32, 64) and st["k"].shape == (256, 8, 128)
    v = synth.bf16_bits_to_f64(st["v"])
    k = synth.bf16_bits_to_f64(st["k"])
    assert abs(v.var() - 1.0) < 0.01 and abs(k.var() * 128 - 1.0) < 0.02
    s0 = synth.state0(sh.with_(batch=2), 1, 1)
    assert abs(s0.var() - 0.1) < 0.002
    g = synth.gdn_round_inputs(synth.WORKLOADS[4].shape.with_(batch=8), 1, 4, 0)
    kk = synth.bf16_bits_to_f64(g["k"])
    assert np.allclose(np.linalg.norm(kk, axis=-1), 1.0, atol=1e-2)
    assert np.all(g["g"] < 0) and np.all((g["beta"] > 0) & (g["beta"] < 1))
    acc = synth.accept_draws(1, 2, 50, 64, 4)
    assert acc.min() == 0 and acc.max() == 4


def test_keyed_streams_are_reproducible_and_distinct():
    sh = synth.WORKLOADS[0].shape
    a = synth.mamba2_step_inputs(sh, 5, 0, 3)
    b = synth.mamba2_step_inputs(sh, 5, 0, 3)
    c = synth.mamba2_step_inputs(sh, 5, 0, 4)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert not np.array_equal(a["v"], c["v"])
    full = synth.state0(sh, 5, 0)
    sub = synth.state0(sh, 5, 0, requests=[2])
    assert np.array_equal(full[2], sub[0])
