"""GPU parity of the per-draft snapshot route (the speculative baseline) and its
device-side commit, through the C ABI, against the CPU oracle's snapshot
semantics on the same seeded inputs.

Slots that hold no committed state are filled with NaN before the first round,
so any read of a slot other than the committed one would show up in y.  Bars as
the other parity tests: y within 1e-3, fp32 state within 1e-4 (tests/util.rel_err);
slot indices and error bits bit-exact."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_amd as rd
from oracle import gdn as o_gdn
from oracle import mamba2 as o_m2
from ssm_recurrent_decode_amd import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, gdn_step_f64, mamba2_step_f64
from tests.util import rel_err

pytestmark = pytest.mark.gpu

Y_TOL, S_TOL = 1e-3, 1e-4


def _dims(sh):
    return rd.Dims(sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity)


def _pool(S0, P, slot0):
    """[B, P, H, d, n] with the committed state in slot slot0[b], NaN elsewhere."""
    B = S0.shape[0]
    pool = torch.full((B, P) + S0.shape[1:], float("nan"), device="cuda")
    for b in range(B):
        pool[b, int(slot0[b])] = dev_f32(S0[b])
    return pool


def _run_rounds(sh, T, P, R, gdn, cfg_id):
    seed = synth.WORKLOADS[cfg_id].cfg_seed
    B = sh.batch
    S0 = synth.state0(sh, seed, cfg_id)
    acc = synth.accept_draws(seed, cfg_id, R, B, T)
    slot0 = np.arange(B) % P
    pool = _pool(S0, P, slot0)
    slot = dev_i32(slot0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty(B, T, sh.nheads, sh.head_dim, device="cuda")
    dims = _dims(sh)
    S = S0.astype(np.float64)
    cur = slot0.copy()
    if not gdn:
        A, dt_bias = synth.mamba2_head_params(sh, seed, cfg_id)
    for r in range(R):
        before = pool.clone()
        if gdn:
            st = synth.gdn_round_inputs(sh, seed, cfg_id, r)
            rd.gdn_snapshot_verify_T(dims, T, pool, slot, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                     dev_bf16(st["q"]), dev_f32(st["g"]), dev_f32(st["beta"]), y, err)
            y_ref, S = o_gdn.spec_round_snapshot(S, gdn_step_f64(st), sh.ngroups, acc[r])
        else:
            st = synth.mamba2_step_inputs(sh, seed, cfg_id, r)
            if T == 1:                      # the generator drops the draft axis at T = 1
                st = {k_: v_[:, None] for k_, v_ in st.items()}
            rd.ssm_snapshot_verify_T(dims, T, pool, slot, dev_bf16(st["v"]), dev_bf16(st["k"]),
                                     dev_bf16(st["q"]), dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A),
                                     y, err)
            y_ref, S = o_m2.spec_round_snapshot(S, mamba2_step_f64(st), dt_bias.astype(np.float64),
                                                A.astype(np.float64), sh.ngroups, acc[r])
        e = rel_err(y.cpu().numpy(), y_ref)
        assert e <= Y_TOL, (r, e)
        # slots outside the committed one and the T after it are untouched
        for b in range(B):
            written = {(int(cur[b]) + i) % P for i in range(T + 1)}
            for s_ in set(range(P)) - written:
                assert torch.equal(pool[b, s_].isnan(), before[b, s_].isnan()), (r, b, s_)
                assert torch.equal(torch.nan_to_num(pool[b, s_]), torch.nan_to_num(before[b, s_]))
        rd.snapshot_commit(T, P, slot, dev_i32(acc[r]), err)
        cur = (cur + acc[r]) % P
        assert slot.cpu().numpy().tolist() == cur.tolist(), r
        got = pool[torch.arange(B, device="cuda"), slot.long()].cpu().numpy()
        es = rel_err(got, S)
        assert es <= S_TOL, (r, es)
    assert int(err.item()) == 0


@pytest.mark.parametrize("d,G,T,extra", [(64, 1, 4, 0), (64, 2, 1, 1), (128, 4, 3, 0), (64, 1, 6, 2),
                                         (128, 2, 8, 0)])
def test_ssm_snapshot_verify_commit_small(d, G, T, extra):
    """Mamba-2: y of every draft (rejected included) and the committed snapshot
    after every commit, over rounds with seeded acceptance draws."""
    sh = synth.WORKLOADS[2].shape.with_(batch=5, head_dim=d, ngroups=G, T=T)
    _run_rounds(sh, T, T + 1 + extra, 12, gdn=False, cfg_id=2)


@pytest.mark.parametrize("d,n,G,T", [(64, 64, 1, 4), (128, 64, 2, 3), (64, 256, 2, 2), (128, 256, 1, 6)])
def test_ssm_snapshot_state_sizes(d, n, G, T):
    """Mamba-2 snapshot route at state sizes 64 and 256."""
    sh = synth.WORKLOADS[2].shape.with_(batch=3, nheads=4, head_dim=d, state_dim=n, ngroups=G, T=T)
    _run_rounds(sh, T, T + 2, 8, gdn=False, cfg_id=2)


@pytest.mark.parametrize("d,G,T,extra", [(128, 32, 4, 0), (64, 8, 2, 1), (128, 16, 6, 0), (64, 4, 8, 0)])
def test_gdn_snapshot_verify_commit_small(d, G, T, extra):
    sh = synth.WORKLOADS[4].shape.with_(batch=3, head_dim=d, ngroups=G, T=T)
    _run_rounds(sh, T, T + 1 + extra, 12, gdn=True, cfg_id=4)


def test_snapshot_anomalies_are_clamped_and_flagged():
    sh = synth.WORKLOADS[2].shape.with_(batch=4, T=2)
    T, P, B = 2, 3, 4
    dims = _dims(sh)
    seed = synth.WORKLOADS[2].cfg_seed
    A, dt_bias = synth.mamba2_head_params(sh, seed, 2)
    S0 = synth.state0(sh, seed, 2)
    pool = _pool(S0, P, np.zeros(B, int))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    slot = dev_i32(np.zeros(B, int))
    rd.snapshot_commit(T, P, slot, dev_i32(np.array([3, -1, 2, 1])), err)
    assert int(err.item()) == 2                       # accepted outside [0, T]
    assert slot.cpu().tolist() == [2, 0, 2, 1]
    err.zero_()
    slot = dev_i32(np.array([P, -1, 0, 2 * P + 1]))   # committed slot out of range
    st = synth.mamba2_step_inputs(sh, seed, 2, 0)
    y = torch.empty(B, T, sh.nheads, sh.head_dim, device="cuda")
    pool[:, :] = dev_f32(S0)[:, None]
    rd.ssm_snapshot_verify_T(dims, T, pool, slot, dev_bf16(st["v"]), dev_bf16(st["k"]), dev_bf16(st["q"]),
                             dev_f32(st["dt"]), dev_f32(dt_bias), dev_f32(A), y, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert torch.isfinite(y).all()
    err.zero_()
    rd.snapshot_commit(T, P, slot, dev_i32(np.zeros(B, int)), err)
    assert int(err.item()) == 1
    assert slot.cpu().tolist() == [0, 2, 0, 1]
