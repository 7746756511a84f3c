"""The C ABI from C++ without Python: tests/c_abi/abi_roundtrip (built with the
library) allocates with hipMalloc, drives the standard step and ReplaySSM
append-decode on one HIP stream, and checks that the outputs agree and that the
pointer word follows the flush-when-full schedule.  Run as a child process; it
also writes the inputs it generated and the outputs it got back, which are then
compared with the float64 oracle's recurrence (every step, both entry points)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import mamba2 as om  # noqa: E402
from tests.util import rel_err  # noqa: E402

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_roundtrip")
# the sizes the program runs (batch, heads, head dim, state, groups, capacity, steps)
B, H, D, N, G, L = 4, 8, 64, 128, 2, 8
STEPS = 2 * L + 3


def _bf16(path, shape):
    bits = np.fromfile(path, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64).reshape(shape)


def _f32(path, shape):
    return np.fromfile(path, dtype=np.float32).astype(np.float64).reshape(shape)


def test_c_program_drives_the_abi(tmp_path):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with `python -m ssm_recurrent_decode_amd.build`")
    print(f"[c_abi] {EXE} {tmp_path}", flush=True)
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout

    S0 = _f32(tmp_path / "S0.f32", (B, H, D, N))
    A = _f32(tmp_path / "A.f32", (H,))
    bias = _f32(tmp_path / "dt_bias.f32", (H,))
    v = _bf16(tmp_path / "v.bf16", (STEPS, B, H, D))
    k = _bf16(tmp_path / "k.bf16", (STEPS, B, G, N))
    q = _bf16(tmp_path / "q.bf16", (STEPS, B, G, N))
    dt = _f32(tmp_path / "dt.f32", (STEPS, B, H))
    y_rep = _f32(tmp_path / "y_replay.f32", (STEPS, B, H, D))
    y_std = _f32(tmp_path / "y_standard.f32", (STEPS, B, H, D))
    steps = [{"v": v[t], "k": k[t], "q": q[t], "dt": dt[t]} for t in range(STEPS)]
    ys, _ = om.run_standard(S0, steps, bias, A, G)
    for t in range(STEPS):
        assert rel_err(y_rep[t], ys[t]) < 1e-3, ("replay_append_decode", t)
        assert rel_err(y_std[t], ys[t]) < 1e-3, ("ssm_decode_step", t)
