"""Helpers for the GPU parity tests: moving generator output to the device and
building oracle sub-problems for sampled (request, head) pairs.

Sampling is exact: requests and heads are independent, so the oracle run on a
subset of (b, h) pairs -- each as its own pseudo-request with one head and one
group -- computes exactly those outputs of the full problem."""
from __future__ import annotations

import numpy as np
import torch

from ssm_recurrent_decode_amd import synth

DEV = "cuda"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_i32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def f64(bits_or_f32, bf16: bool) -> np.ndarray:
    return synth.bf16_bits_to_f64(bits_or_f32) if bf16 else np.asarray(bits_or_f32, np.float64)


def mamba2_step_f64(st: dict) -> dict:
    return {"v": f64(st["v"], True), "k": f64(st["k"], True), "q": f64(st["q"], True),
            "dt": f64(st["dt"], False)}


def gdn_step_f64(st: dict) -> dict:
    return {"v": f64(st["v"], True), "k": f64(st["k"], True), "q": f64(st["q"], True),
            "g": f64(st["g"], False), "beta": f64(st["beta"], False)}


def sample_pairs(B: int, H: int, n: int, seed: int):
    """(b, h) pairs covering the first/last request and head plus seeded picks."""
    rng = np.random.default_rng(seed)
    fixed = [(0, 0), (B - 1, H - 1), (B // 2, H // 2), (0, H - 1), (B - 1, 0)]
    pairs = list(dict.fromkeys(fixed))
    while len(pairs) < n:
        p = (int(rng.integers(B)), int(rng.integers(H)))
        if p not in pairs:
            pairs.append(p)
    return pairs[:n]


def every_request_pairs(B: int, H: int, per: int = 2):
    """``per`` heads of every request, rotating so that the heads taken over all
    requests cover every head: (b, (b + j H / per) mod H) for j < per."""
    return [(b, (b + j * (H // per)) % H) for b in range(B) for j in range(per)]


def sub_mamba2(pairs, H, G, st: dict, spec: bool = False) -> dict:
    """Slice one step's (or round's) float64 inputs to pseudo-requests (b, h):
    one head and one group each."""
    hpg = H // G
    bi = np.array([b for b, _ in pairs])
    hi = np.array([h for _, h in pairs])
    gi = hi // hpg
    if not spec:
        return {"v": st["v"][bi, hi][:, None], "k": st["k"][bi, gi][:, None],
                "q": st["q"][bi, gi][:, None], "dt": st["dt"][bi, hi][:, None]}
    return {"v": st["v"][bi, :, hi][:, :, None], "k": st["k"][bi, :, gi][:, :, None],
            "q": st["q"][bi, :, gi][:, :, None], "dt": st["dt"][bi, :, hi][:, :, None]}


def sub_gdn(pairs, H, G, st: dict) -> dict:
    hpg = H // G
    bi = np.array([b for b, _ in pairs])
    hi = np.array([h for _, h in pairs])
    gi = hi // hpg
    return {"v": st["v"][bi, :, hi][:, :, None], "k": st["k"][bi, :, gi][:, :, None],
            "q": st["q"][bi, :, gi][:, :, None], "g": st["g"][bi, :, hi][:, :, None],
            "beta": st["beta"][bi, :, hi][:, :, None]}


def pair_index(pairs):
    bi = torch.tensor([b for b, _ in pairs], device=DEV)
    hi = torch.tensor([h for _, h in pairs], device=DEV)
    return bi, hi
