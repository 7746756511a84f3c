#!/usr/bin/env python3
"""Decode throughput of one Nemotron-H-like SSM layer on one MI355X.

Workload (one "step"): one decode token for every request of the batch through
one SSM layer -- the fused causal conv1d state update (conv state 3072 x 3 bf16,
width 4, SiLU) followed by ReplaySSM append-decode (batch 256, 32 heads, head dim
64, state 128, 8 groups, ring capacity 16: step size and decay, ring append,
decay-prefix weights, shared k.q inner products, checkpoint read S_0 q, output
combine, and the fused flush on every 16th step).  Inputs are seeded synthetic
tensors with the workload's distributions, resident in device memory before the
timed region; consecutive steps rotate over several independent layer instances
(checkpoint + ring + conv state each) so the working set exceeds the 256 MB
Infinity Cache and the state is streamed from HBM.

Prints ONE JSON line.  `value` is decode tokens/s of the layer (batch x steps /
time), from the median of at least 20 timed replays of a HIP graph holding one
ring cycle of every rotated layer (flush steps included).  `roofline` is for the
dominant kernel, replay_append_decode: algorithmic bytes per launch averaged over
whole ring cycles / its average launch duration over those launches, measured
with HIP events on its stream, against the 8 TB/s HBM peak; flush and non-flush
launches are also reported separately.  `cpu_baseline` is the CPU oracle
(ReplaySSM bookkeeping in float64 numpy) timed on a bounded sample of the same
workload, with the host's CPU model and core count.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
import traceback

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def _args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--layers", type=int, default=4, help="layer instances rotated per step")
    ap.add_argument("--pool", type=int, default=32, help="distinct pre-generated step inputs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-standard", action="store_true", help="skip the standard-step comparator")
    ap.add_argument("--cpu-steps", type=int, default=96,
                    help="decode steps of the CPU oracle sample (96: about 10 s on one core)")
    ap.add_argument("--no-graph", action="store_true",
                    help="no HIP graphs: the step eagerly only, and the rows without their graph passes "
                         "(so that hardware counters see only launches whose bytes the rows account exactly)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other measured rows (verify, GDN verify, capacity sweep)")
    ap.add_argument("--rows", default=None,
                    help="comma-separated subset of the rows to run (default: all)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the 1 GiB copy probe (for scaling traffic counters) and exit")
    return ap.parse_args(argv)


def _calibrate_copy():
    """Eight launches of the streaming copy probe over 1 GiB: each reads and writes
    exactly 2^30 bytes, so FETCH_SIZE / WRITE_SIZE of these dispatches give the
    counters' scale."""
    import torch
    import ssm_recurrent_decode_amd as rd
    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(8):
        rd.rssm_probe_copy(dst, src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "rssm_probe_copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 8}))


def _ceiling_probes(torch, rd, dev, stream, launch_bytes):
    """This part's streaming ceilings, measured in the same process: the read probe
    over one launch's checkpoint bytes (four buffers rotated, so nothing stays in
    the 256 MB Infinity Cache) and over 1 GiB, and the 1 GiB copy probe (read +
    write).  16 back-to-back launches under one HIP event pair, as the kernels
    are timed; then the same 16 with an event pair around each launch (the mean,
    `us_event_pair_each`: that adds the gap between launches to every one)."""
    res = {}
    for name, nbytes, nbuf, copy in (("read_one_launch", launch_bytes, 4, False),
                                     ("read_1GiB", 1 << 30, 1, False), ("copy_1GiB", 1 << 30, 1, True)):
        nbytes -= nbytes % 16
        bufs = [torch.empty(nbytes // 4, device=dev) for _ in range(nbuf)]
        for b_ in bufs:
            b_.zero_()
        dst = torch.empty_like(bufs[0]) if copy else None
        sink = torch.empty(rd.probe_read_sink_floats(nbytes), device=dev)

        def run(i):
            if copy:
                rd.rssm_probe_copy(dst, bufs[i % nbuf], stream=stream)
            else:
                rd.rssm_probe_read(bufs[i % nbuf], sink, stream=stream)
        for i in range(4):
            run(i)
        ev = _events(torch, 17)
        torch.cuda.synchronize()
        ev[16][0].record(stream)
        for i in range(16):
            run(i)
        ev[16][1].record(stream)
        torch.cuda.synchronize()
        us = 1e3 * ev[16][0].elapsed_time(ev[16][1]) / 16
        for i in range(16):
            ev[i][0].record(stream)
            run(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us_each = sum(1e3 * a_.elapsed_time(b_) for a_, b_ in ev[:16]) / 16
        moved = nbytes * (2 if copy else 1)
        res[name] = {"bytes": moved, "us": round(us, 2), "GBs": round(moved / (us * 1e-6) / 1e9, 1),
                     "us_event_pair_each": round(us_each, 2),
                     "GBs_event_pair_each": round(moved / (us_each * 1e-6) / 1e9, 1)}
        del bufs, dst, sink
    return res


def _cpu_inputs(steps: int, lo: int, hi: int):
    """Requests lo..hi-1 of the headline workload as float64: checkpoint, head
    parameters and `steps` decode steps (the values the GPU receives)."""
    import numpy as np

    from ssm_recurrent_decode_amd import synth
    wl = synth.WORKLOADS[1]
    sh, seed = wl.shape, wl.cfg_seed
    A, bias = synth.mamba2_head_params(sh, seed, 1)
    S0 = synth.state0(sh, seed, 1)[lo:hi].astype(np.float64)
    seq = []
    for t in range(steps):
        st = synth.mamba2_step_inputs(sh, seed, 1, t)
        seq.append({"v": synth.bf16_bits_to_f64(st["v"][lo:hi]), "k": synth.bf16_bits_to_f64(st["k"][lo:hi]),
                    "q": synth.bf16_bits_to_f64(st["q"][lo:hi]), "dt": st["dt"][lo:hi].astype(np.float64)})
    return sh, S0, seq, bias.astype(np.float64), A.astype(np.float64)


def _cpu_worker(job):
    """One process of the all-cores leg: the oracle over its slice of requests,
    started together with the others at a shared barrier; returns its wall-clock
    interval (CLOCK_MONOTONIC is system-wide)."""
    steps, lo, hi, barrier = job
    from oracle import replay as o_rep
    sh, S0, seq, bias, A = _cpu_inputs(steps, lo, hi)
    barrier.wait()
    t0 = time.monotonic()
    o_rep.run_standard(S0, seq, bias, A, sh.capacity, sh.ngroups)
    return t0, time.monotonic()


def _cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _host():
    return {"cpu_model": _cpu_model(), "cores_available": len(os.sched_getaffinity(0))}


def _cpu_baseline(steps: int):
    """The CPU oracle (ReplaySSM standard mode, float64) on the full batch of the
    same workload for `steps` decode steps; single-threaded numpy elementwise code."""
    from oracle import replay as o_rep
    sh, S0, seq, bias, A = _cpu_inputs(steps, 0, None)
    t0 = time.perf_counter()
    o_rep.run_standard(S0, seq, bias, A, sh.capacity, sh.ngroups)
    dt = time.perf_counter() - t0
    return {"value": sh.batch * steps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"ReplaySSM standard-mode oracle, full batch {sh.batch}, {steps} decode steps "
                      f"({steps // sh.capacity} flushes), float64 numpy, {dt:.1f} s", **_host()}


# Worker processes of the all-cores leg: the share of a multi-GPU host's cores
# that one GPU's jobs may use.
CPU_WORKERS_MAX = 16


def _cpu_baseline_all_cores(steps: int, max_workers: int = CPU_WORKERS_MAX):
    """The same oracle on the host cores this process may use, at most
    `max_workers` of them: requests are independent, so the batch is split into
    equal slices, one fresh (spawned) process per slice, all released at once;
    the rate is the whole batch over the span from the first start to the last
    finish."""
    import multiprocessing as mp

    from ssm_recurrent_decode_amd import synth
    B = synth.WORKLOADS[1].shape.batch
    host = _host()
    W = max(1, min(host["cores_available"], max_workers, B))
    cuts = [B * i // W for i in range(W + 1)]
    ctx = mp.get_context("spawn")
    with ctx.Manager() as mgr:
        barrier = mgr.Barrier(W)
        with ctx.Pool(W) as pool:
            spans = pool.map(_cpu_worker, [(steps, cuts[i], cuts[i + 1], barrier) for i in range(W)])
    dt = max(e for _, e in spans) - min(s for s, _ in spans)
    return {"value": B * steps / dt, "unit": "tokens/s", "cores": W, "kind": "oracle",
            "sample": f"the same oracle, full batch {B} split over {W} processes ({W} of the "
                      f"{host['cores_available']} cores this process may use; at most {max_workers}), "
                      f"{steps} decode steps, {dt:.1f} s wall", **host}


def _cpu_standard_baseline(cfg_id: int, requests: int, capacity: int = 16):
    """The standard-mode ReplaySSM oracle (float64, one core) on a bounded sample
    of a decode workload: the first `requests` requests over one ring cycle of
    `capacity` steps (the fold included)."""
    import numpy as np

    from oracle import replay as o_rep
    from ssm_recurrent_decode_amd import synth
    wl = synth.WORKLOADS[cfg_id]
    sh, seed = wl.shape.with_(capacity=capacity), wl.cfg_seed
    n = min(requests, sh.batch)
    A, bias = synth.mamba2_head_params(sh, seed, cfg_id)
    S0 = np.stack([synth.state0_request(sh, seed, cfg_id, b) for b in range(n)]).astype(np.float64)
    seq = []
    for t in range(capacity):
        st = synth.mamba2_step_inputs(sh, seed, cfg_id, t)
        seq.append({"v": synth.bf16_bits_to_f64(st["v"][:n]), "k": synth.bf16_bits_to_f64(st["k"][:n]),
                    "q": synth.bf16_bits_to_f64(st["q"][:n]), "dt": st["dt"][:n].astype(np.float64)})
    t0 = time.perf_counter()
    o_rep.run_standard(S0, seq, bias.astype(np.float64), A.astype(np.float64), capacity, sh.ngroups)
    dt = time.perf_counter() - t0
    return {"value": n * capacity / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"ReplaySSM standard-mode oracle, requests 0..{n - 1} of {sh.batch} ({sh.nheads} heads), "
                      f"{capacity} decode steps (one ring cycle, L = {capacity}), float64 numpy, {dt:.1f} s",
            **_host()}


def _cpu_spec_baseline(cfg_id: int, requests: int, rounds: int = 16):
    """The speculative oracle (float64, one core) on a bounded sample of a verify
    workload: the first `requests` requests of the batch over `rounds` verify
    rounds with the workload's acceptance draws.  Mamba-2: ReplaySSM spec-mode
    bookkeeping; GDN: the committed state rebuilt from the ring, T serial draft
    steps.  Rates are per verified position and per accepted token."""
    import numpy as np

    from oracle import gdn as o_gdn
    from oracle import replay as o_rep
    from ssm_recurrent_decode_amd import synth
    wl = synth.WORKLOADS[cfg_id]
    sh, seed, gdn = wl.shape, wl.cfg_seed, cfg_id == 4
    n, T = min(requests, sh.batch), sh.T
    S0 = np.stack([synth.state0_request(sh, seed, cfg_id, b) for b in range(n)]).astype(np.float64)
    acc = synth.accept_draws(seed, cfg_id, rounds, sh.batch, T)[:, :n]
    seq = []
    for r in range(rounds):
        st = synth.gdn_round_inputs(sh, seed, cfg_id, r) if gdn else synth.mamba2_step_inputs(sh, seed, cfg_id, r)
        seq.append({k: (synth.bf16_bits_to_f64(v[:n]) if v.dtype == np.uint16 else v[:n].astype(np.float64))
                    for k, v in st.items()})
    if gdn:
        reqs = [o_gdn.GDNReplayRequest(S0[b], sh.capacity, sh.ngroups) for b in range(n)]
        t0 = time.perf_counter()
        for r, rd_ in enumerate(seq):
            for b, q in enumerate(reqs):
                q.verify_round(rd_["v"][b], rd_["k"][b], rd_["q"][b], rd_["g"][b], rd_["beta"][b])
                q.commit(int(acc[r, b]))
        dt = time.perf_counter() - t0
    else:
        A, bias = synth.mamba2_head_params(sh, seed, cfg_id)
        t0 = time.perf_counter()
        o_rep.run_spec(S0, seq, bias.astype(np.float64), A.astype(np.float64), sh.capacity, sh.ngroups, acc)
        dt = time.perf_counter() - t0
    return {"value": n * T * rounds / dt, "unit": "verified positions/s",
            "accepted_tokens_per_s": float(acc.sum()) / dt, "cores": 1, "kind": "oracle",
            "sample": f"{'GDN' if gdn else 'Mamba-2'} speculative oracle, requests 0..{n - 1} of {sh.batch}, "
                      f"{rounds} verify rounds of T={T}, float64 numpy, {dt:.1f} s", **_host()}


# ------------------------------------------------------------------ other rows
def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def _verify_bytes(traffic, gdn, H, D, N, G, T, L, counts, flags=0):
    """Algorithmic bytes of one verify launch from the committed counts the
    kernel saw (one per request); flags select bf16 y / bf16 GDN corrections."""
    yb = 2 if flags & 1 else 4
    tot = 0
    for c in set(int(x) for x in counts):
        nb = int((counts == c).sum())
        if gdn:
            tot += traffic.gdn_verify(nb, H, D, N, G, T, c, c + 2 * T > L, yb, 2 if flags & 2 else 4)
        else:
            tot += traffic.replay_verify(nb, H, D, N, G, T, c, c + 2 * T > L, yb)
    return tot


def _draft_inputs(synth, sh, seed, cfg_id, r, gdn):
    """One verify round of seeded draft inputs with the draft axis kept at T = 1."""
    if gdn:
        return synth.gdn_round_inputs(sh, seed, cfg_id, r)
    st = synth.mamba2_step_inputs(sh, seed, cfg_id, r)
    return {k_: v_[:, None] for k_, v_ in st.items()} if sh.T == 1 else st


# Whether the rows also time their HIP-graph passes (off under --no-graph).
ROW_GRAPHS = True


def _row_verify(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, rounds=64, warm=48, T=None,
                with_standard=True, flags=0, G=None, shape=None, light=False):
    """Speculative verify rounds (verify kernel + device-side rollback) on two
    rotated layer instances.  A first pass records the committed count every
    request had before each round; the rings are reset and the same sequence is
    replayed with HIP events around every launch.  T and G override the
    workload's draft window and group count, `shape` any other of its sizes;
    `light` times the verify rounds only (no commit-and-verify pass, no
    fixed-pointer rounds, no standard step).  The first `warm` rounds of each
    pass are not timed: after a pause of the stream (the host reading the
    pointers, the rings reset between passes) the first few milliseconds of
    rounds run up to 15 % slower on this part.
    """
    wl = synth.WORKLOADS[cfg_id]
    sh, seed = (wl.shape if T is None else wl.shape.with_(T=T)), wl.cfg_seed
    if G is not None:
        sh = sh.with_(ngroups=G)
    if shape:
        sh = sh.with_(**shape)
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    NLr, P, R = 2, 8, warm + rounds
    dims = rd.Dims(B, H, D, N, G, L, flags=flags)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    gen = torch.Generator(device=dev)
    layers = []
    for l in range(NLr):
        gen.manual_seed(seed * 100 + l)
        Ly = {"S0": torch.randn((B, H, D, N), generator=gen, device=dev) * math.sqrt(0.1),
              "ring": rd.Ring(dims, gdn=gdn, device=dev)}
        if not gdn:
            A, bias = synth.mamba2_head_params(sh, seed, cfg_id, layer=l)
            Ly["A"], Ly["bias"] = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
        layers.append(Ly)
    pool = []
    for p in range(P):
        st = _draft_inputs(synth, sh, seed, cfg_id, p, gdn)
        pool.append({k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(v_)).to(dev))
                     for k_, v_ in st.items()})
    acc = synth.accept_draws(seed, cfg_id, R, B, T)
    dacc = [torch.from_numpy(acc[r]).to(dev) for r in range(R)]
    y = torch.empty((B, T, H, D), dtype=torch.bfloat16 if flags & 1 else torch.float32, device=dev)
    flushed = torch.zeros((B,), dtype=torch.int32, device=dev)

    def verify(r):
        Ly, ip = layers[r % NLr], pool[r % P]
        if gdn:
            rd.gdn_replay_verify_T(dims, T, Ly["S0"], Ly["ring"], ip["v"], ip["k"], ip["q"], ip["g"],
                                   ip["beta"], y, flushed, stream=stream)
        else:
            rd.replay_verify_T(dims, T, Ly["S0"], Ly["ring"], ip["v"], ip["k"], ip["q"], ip["dt"],
                               Ly["bias"], Ly["A"], y, flushed, stream=stream)

    def rollback(r):
        rd.replay_rollback(dims, layers[r % NLr]["ring"], dacc[r], stream=stream)

    counts = []
    for r in range(R):                       # pass 1: pointers each round saw
        torch.cuda.synchronize()
        counts.append(layers[r % NLr]["ring"].count.cpu().numpy().copy())
        verify(r)
        rollback(r)
    torch.cuda.synchronize()
    for Ly in layers:
        rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
    ev_v, ev_r = _events(torch, R), _events(torch, R)
    torch.cuda.synchronize()
    for r in range(R):                       # pass 2: the same rounds, timed
        ev_v[r][0].record(stream)
        verify(r)
        ev_v[r][1].record(stream)
        rollback(r)
        ev_r[r][1].record(stream)
    torch.cuda.synchronize()
    errs = [int(Ly["ring"].err.item()) for Ly in layers]
    if any(errs):
        raise RuntimeError(f"ring anomaly bits set: {errs}")
    v_us = [1e3 * ev_v[r][0].elapsed_time(ev_v[r][1]) for r in range(warm, R)]
    r_us = [1e3 * ev_v[r][1].elapsed_time(ev_r[r][1]) for r in range(warm, R)]
    byts = [_verify_bytes(traffic, gdn, H, D, N, G, T, L, counts[r], flags) for r in range(warm, R)]
    fl = np.array([counts[r] + 2 * T > L for r in range(warm, R)])
    round_s = (sum(v_us) + sum(r_us)) * 1e-6
    gbs = sum(byts) / (sum(v_us) * 1e-6) / 1e9
    if light:
        return {"batch": B, "nheads": H, "head_dim": D, "state_dim": N, "ngroups": G, "capacity": L, "T": T,
                "verify_us": round(sum(v_us) / rounds, 3), "achieved_GBs": round(gbs, 1),
                "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_round": round(sum(byts) / rounds),
                "flush_rate": round(float(fl.mean()), 4)}
    # the same rounds with each commit folded into the next verify launch
    # (commit-and-verify: one launch per round; the last window's commit is the
    # separate kernel, outside the timed rounds)
    for Ly in layers:
        rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
    zero = torch.zeros((B,), dtype=torch.int32, device=dev)
    ev_c = _events(torch, R)
    torch.cuda.synchronize()
    for r in range(R):
        Ly, ip = layers[r % NLr], pool[r % P]
        prev = dacc[r - NLr] if r >= NLr else zero       # this ring's previous window
        ev_c[r][0].record(stream)
        if gdn:
            rd.gdn_replay_commit_verify_T(dims, T, Ly["S0"], Ly["ring"], prev, ip["v"], ip["k"], ip["q"], ip["g"],
                                          ip["beta"], y, flushed, stream=stream)
        else:
            rd.replay_commit_verify_T(dims, T, Ly["S0"], Ly["ring"], prev, ip["v"], ip["k"], ip["q"], ip["dt"],
                                      Ly["bias"], Ly["A"], y, flushed, stream=stream)
        ev_c[r][1].record(stream)
    for l in range(NLr):
        rd.replay_rollback(dims, layers[(R - NLr + l) % NLr]["ring"], dacc[R - NLr + l], stream=stream)
    torch.cuda.synchronize()
    errs = [int(Ly["ring"].err.item()) for Ly in layers]
    if any(errs):
        raise RuntimeError(f"ring anomaly bits set in the commit-and-verify rounds: {errs}")
    cv_us = [1e3 * ev_c[r][0].elapsed_time(ev_c[r][1]) for r in range(warm, R)]
    cv_s = sum(cv_us) * 1e-6
    # the same rounds once more, one event pair around the timed rounds (no events
    # between launches)
    for Ly in layers:
        rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
    blk = _events(torch, 1)[0]
    torch.cuda.synchronize()
    for r in range(R):
        Ly, ip = layers[r % NLr], pool[r % P]
        prev = dacc[r - NLr] if r >= NLr else zero
        if r == warm:
            blk[0].record(stream)
        if gdn:
            rd.gdn_replay_commit_verify_T(dims, T, Ly["S0"], Ly["ring"], prev, ip["v"], ip["k"], ip["q"], ip["g"],
                                          ip["beta"], y, flushed, stream=stream)
        else:
            rd.replay_commit_verify_T(dims, T, Ly["S0"], Ly["ring"], prev, ip["v"], ip["k"], ip["q"], ip["dt"],
                                      Ly["bias"], Ly["A"], y, flushed, stream=stream)
    blk[1].record(stream)
    for l in range(NLr):
        rd.replay_rollback(dims, layers[(R - NLr + l) % NLr]["ring"], dacc[R - NLr + l], stream=stream)
    torch.cuda.synchronize()
    cv_block_us = 1e3 * blk[0].elapsed_time(blk[1]) / rounds
    # the graph timing protocol for the speculative workloads: 16 rounds
    # of commit-and-verify (both layers alternating) captured once in a HIP graph,
    # 5 untimed replays, then 20 timed ones (median and minimum per round); the
    # graph keeps replaying the same accepted counts while the rings move on
    GR = 16
    g_us = _verify_graph_pass(torch, rd, dims, T, gdn, layers, pool, dacc, y, flushed, stream, NLr, P, GR) \
        if ROW_GRAPHS else None
    fixed = _fixed_pointer_rounds(torch, np, rd, traffic, stream, layers, pool, verify, y, dims, gdn, flags)
    # every launch of the kernel in this row: the counting pass, the timed verify
    # pass and the two commit-and-verify passes replay rounds 0..R-1, then the
    # fixed-pointer rounds
    all_bytes = 4 * sum(_verify_bytes(traffic, gdn, H, D, N, G, T, L, counts[r], flags) for r in range(R))
    all_launches = 4 * R
    if g_us is not None:
        # the graph pass (counts not recorded): its launches at the timed pass's mean bytes
        all_bytes += (GR + GR * 25) * sum(byts) / rounds
        all_launches += GR + GR * 25
    for f_ in (fixed or {}).values():
        all_bytes += f_["launches"] * f_["alg_bytes"]
        all_launches += f_["launches"]
    base = None
    if gdn and with_standard:
        # the baseline that rewrites the state every token, at the same shape
        base = _standard_step_row(torch, np, rd, synth, traffic, dev, stream, cfg_id, True,
                                  [Ly["S0"] for Ly in layers])
    cv = {"kernel": "gdn_replay_commit_verify_T" if gdn else "replay_commit_verify_T",
          "us_per_round": round(sum(cv_us) / rounds, 3),
          "verified_positions_per_s": round(B * T * rounds / cv_s, 1),
          "accepted_tokens_per_s": round(float(acc[warm:].sum()) / cv_s, 1),
          "achieved_GBs": round(sum(byts) / cv_s / 1e9, 1),
          "us_per_round_block": round(cv_block_us, 3),
          "achieved_GBs_block": round(sum(byts) / (cv_block_us * rounds * 1e-6) / 1e9, 1)}
    if g_us is not None:
        cv["graph"] = {"rounds_per_replay": GR, "replays_timed": 20, "warmup_replays": 5,
                       "us_per_round_median": round(g_us[10], 3),
                       "us_per_round_min": round(g_us[0], 3),
                       "verified_positions_per_s": round(B * T / (g_us[10] * 1e-6), 1),
                       "achieved_GBs": round(sum(byts) / rounds / (g_us[10] * 1e-6) / 1e9, 1),
                       "bytes_note": "mean algorithmic bytes per round of the timed pass"}
    res = {"workload": ("Gated DeltaNet" if gdn else "Mamba-2") +
                       f" speculative verify, batch {B}, {H} heads, head dim {D}, state {N}, "
                       f"{G} group(s), ring capacity {L}, T={T}; two layer instances rotated",
           "kernel": "gdn_replay_verify_T" if gdn else "replay_verify_T",
           "rounds_timed": rounds, "verify_us": round(sum(v_us) / rounds, 3),
           "rollback_us": round(sum(r_us) / rounds, 3),
           "verified_positions_per_s": round(B * T * rounds / round_s, 1),
           "accepted_tokens_per_s": round(float(acc[warm:].sum()) / round_s, 1),
           "achieved_GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
           "alg_bytes_per_round": round(sum(byts) / rounds),
           # over every launch of the kernel (four passes replay rounds 0..R-1, the
           # graph pass, then the fixed-pointer rounds): the figure hardware traffic
           # counters over the whole run compare with
           "alg_bytes_avg_all_launches": round(all_bytes / all_launches),
           "launches": all_launches,
           "flush_rate": round(float(fl.mean()), 4),
           "commit_verify": cv,
           "mean_committed_before": round(float(np.mean([counts[r] for r in range(warm, R)])), 3)}
    if fixed is not None:
        res["fixed_pointer_rounds"] = fixed
    if base is not None:
        res["standard_step"] = base
    return res


def _verify_graph_pass(torch, rd, dims, T, gdn, layers, pool, dacc, y, flushed, stream, NLr, P, GR):
    """The commit-and-verify rounds under the graph protocol; per-round times of
    the 20 timed replays, sorted."""
    for Ly in layers:
        rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
    torch.cuda.synchronize()

    def cv_round(r):
        Ly, ip = layers[r % NLr], pool[r % P]
        prev = dacc[(r - NLr) % GR]
        if gdn:
            rd.gdn_replay_commit_verify_T(dims, T, Ly["S0"], Ly["ring"], prev, ip["v"], ip["k"], ip["q"], ip["g"],
                                          ip["beta"], y, flushed, stream=stream)
        else:
            rd.replay_commit_verify_T(dims, T, Ly["S0"], Ly["ring"], prev, ip["v"], ip["k"], ip["q"], ip["dt"],
                                      Ly["bias"], Ly["A"], y, flushed, stream=stream)
    for r in range(GR):                     # untimed: fills the rings to the stationary mix
        cv_round(r)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for r in range(GR):
            cv_round(r)
    ev_g = _events(torch, 20)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        for _ in range(5):
            graph.replay()
        for i in range(20):
            ev_g[i][0].record(stream)
            graph.replay()
            ev_g[i][1].record(stream)
    torch.cuda.synchronize()
    g_us = sorted(1e3 * a_.elapsed_time(b_) / GR for a_, b_ in ev_g)
    errs = [int(Ly["ring"].err.item()) for Ly in layers]
    if any(errs):
        raise RuntimeError(f"ring anomaly bits set in the graph-replayed rounds: {errs}")
    for Ly in layers:
        rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
    torch.cuda.synchronize()
    return g_us


def _fixed_pointer_rounds(torch, np, rd, traffic, stream, layers, pool, verify, y, dims, gdn, flags,
                          reps=24):
    """The verify kernel with every request at the same committed count, so that
    no request folds (c = L - 2T, the largest count that does not) or every one
    does (c = L - T, the largest count a round can start from): the fold's cost
    separated from the rest of a round.  Before each timed launch the pointer
    words of every record are set on the stream (head 0, pending 0, the ring
    slots still hold earlier rounds' entries); events bracket the verify launch
    alone, which folds the c entries (or not) exactly as in a mixed round."""
    B, H, D, N, G, L = dims.batch, dims.nheads, dims.head_dim, dims.state_dim, dims.ngroups, dims.capacity
    T = int(y.shape[1])
    if L < 2 * T or L - 2 * T == L - T:
        return None
    out = {}
    for tag, c in (("no_fold", L - 2 * T), ("all_fold", L - T)):
        word = c << 16                      # head 0, count c, pending 0
        ev = _events(torch, reps)
        torch.cuda.synchronize()
        for i in range(reps):
            Ly = layers[i % len(layers)]
            with torch.cuda.stream(stream):
                Ly["ring"].meta.view(torch.int64)[:, :, 0].fill_(word)
            ev[i][0].record(stream)
            verify(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = sorted(1e3 * a_.elapsed_time(b_) for a_, b_ in ev[4:])
        med = us[len(us) // 2]
        nbytes = _verify_bytes(traffic, gdn, H, D, N, G, T, L, np.full(B, c), flags)
        out[tag] = {"committed_count": c, "folds": c + 2 * T > L, "median_us": round(med, 3),
                    "min_us": round(us[0], 3), "alg_bytes": nbytes, "launches": reps,
                    "achieved_GBs": round(nbytes / (med * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    for Ly in layers:
        rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
    torch.cuda.synchronize()
    return out


def _standard_step_row(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, states, reps=16, shape=None):
    """One-token standard decode (state read and rewritten) at a workload's shape
    (or the given one), rotated over the given state tensors; mean of per-launch
    HIP-event times."""
    wl = synth.WORKLOADS[cfg_id]
    sh, seed = (wl.shape if shape is None else shape).with_(T=1), wl.cfg_seed
    B, H, D, N, G = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups
    dims = rd.Dims(B, H, D, N, G, sh.capacity)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    y1 = torch.empty((B, H, D), device=dev)
    if gdn:
        st = synth.gdn_round_inputs(sh, seed, cfg_id, 0)
        one = {k_: (bf(v_[:, 0]) if v_.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(v_[:, 0])).to(dev))
               for k_, v_ in st.items()}

        def call(i):
            rd.gdn_decode_step(dims, states[i % len(states)], one["v"], one["k"], one["q"], one["g"],
                               one["beta"], y1, stream=stream)
        name, byts = "gdn_decode_step", traffic.gdn_standard_step(B, H, D, N, G)
    else:
        st = synth.mamba2_step_inputs(sh, seed, cfg_id, 0)
        A, bias = synth.mamba2_head_params(sh, seed, cfg_id)
        one = {k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(v_).to(dev)) for k_, v_ in st.items()}
        A, bias = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)

        def call(i):
            rd.ssm_decode_step(dims, states[i % len(states)], one["v"], one["k"], one["q"], one["dt"], bias, A,
                               y1, stream=stream)
        name, byts = "ssm_decode_step", traffic.standard_step(B, H, D, N, G)
    for i in range(4):
        call(i)
    ev = _events(torch, reps)
    torch.cuda.synchronize()
    for i in range(reps):
        ev[i][0].record(stream)
        call(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    su = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in ev]))
    return {"kernel": name, "us": round(su, 3), "GBs": round(byts / (su * 1e-6) / 1e9, 1),
            "tokens_per_s": round(B / (su * 1e-6), 1), "alg_bytes": byts, "launches": 4 + reps}


def _snapshot_rounds(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, T, rounds, warm):
    """The per-draft snapshot route (verify + device-side commit) at a workload's
    shape with window T, on two rotated layer instances of T + 1 state slots per
    request; per-launch HIP-event times."""
    wl = synth.WORKLOADS[cfg_id]
    sh, seed = wl.shape.with_(T=T), wl.cfg_seed
    B, H, D, N, G = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups
    NLr, P, R, nslots = 2, 8, warm + rounds, T + 1
    dims = rd.Dims(B, H, D, N, G, sh.capacity)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    gen = torch.Generator(device=dev)
    layers = []
    for l in range(NLr):
        gen.manual_seed(seed * 100 + l)
        pool_l = torch.empty((B, nslots, H, D, N), device=dev)
        pool_l[:, 0] = torch.randn((B, H, D, N), generator=gen, device=dev) * math.sqrt(0.1)
        layers.append({"pool": pool_l, "slot": torch.zeros((B,), dtype=torch.int32, device=dev)})
        if not gdn:
            A, bias = synth.mamba2_head_params(sh, seed, cfg_id, layer=l)
            layers[-1]["A"], layers[-1]["bias"] = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
    ins = []
    for p in range(P):
        st = _draft_inputs(synth, sh, seed, cfg_id, p, gdn)
        ins.append({k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(v_)).to(dev))
                    for k_, v_ in st.items()})
    acc = synth.accept_draws(seed, cfg_id, R, B, T)
    dacc = [torch.from_numpy(acc[r]).to(dev) for r in range(R)]
    y = torch.empty((B, T, H, D), device=dev)
    err = torch.zeros((1,), dtype=torch.int32, device=dev)
    ev_v, ev_c = _events(torch, R), _events(torch, R)
    torch.cuda.synchronize()
    for r in range(R):
        Ly, ip = layers[r % NLr], ins[r % P]
        ev_v[r][0].record(stream)
        if gdn:
            rd.gdn_snapshot_verify_T(dims, T, Ly["pool"], Ly["slot"], ip["v"], ip["k"], ip["q"], ip["g"],
                                     ip["beta"], y, err, stream=stream)
        else:
            rd.ssm_snapshot_verify_T(dims, T, Ly["pool"], Ly["slot"], ip["v"], ip["k"], ip["q"], ip["dt"],
                                     Ly["bias"], Ly["A"], y, err, stream=stream)
        ev_v[r][1].record(stream)
        rd.snapshot_commit(T, nslots, Ly["slot"], dacc[r], err, stream=stream)
        ev_c[r][1].record(stream)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError("snapshot route anomaly bits set")
    v_us = [1e3 * ev_v[r][0].elapsed_time(ev_v[r][1]) for r in range(warm, R)]
    c_us = [1e3 * ev_v[r][1].elapsed_time(ev_c[r][1]) for r in range(warm, R)]
    byts = traffic.snapshot_verify(B, H, D, N, G, T, gdn)
    us = sum(v_us) / rounds
    return {"kernel": "gdn_snapshot_verify_T" if gdn else "ssm_snapshot_verify_T", "verify_us": round(us, 3),
            "commit_us": round(sum(c_us) / rounds, 3), "achieved_GBs": round(byts / (us * 1e-6) / 1e9, 1),
            "alg_bytes_per_round": byts, "launches": R}


def _row_precision(torch, np, rd, synth, traffic, dev, stream):
    """The speculative verify rows again with the storage-precision options of the
    method page's serving setup: bf16 outputs (Mamba-2), bf16 outputs and bf16
    cached corrections (GDN); per round, against the default fp32 storage."""
    out = {}
    for name, cid, gdn, flags in (("mamba2_y_bf16", 2, False, 1), ("gdn_y_u_bf16", 4, True, 3)):
        base = _row_verify(torch, np, rd, synth, traffic, dev, stream, cid, gdn, rounds=32, warm=8,
                           with_standard=False)
        var = _row_verify(torch, np, rd, synth, traffic, dev, stream, cid, gdn, rounds=32, warm=8,
                          with_standard=False, flags=flags)
        out[name] = {"workload": var["workload"], "flags": flags,
                     "default_verify_us": base["verify_us"], "verify_us": var["verify_us"],
                     "speedup": round(base["verify_us"] / var["verify_us"], 3),
                     "alg_bytes_per_round": var["alg_bytes_per_round"], "achieved_GBs": var["achieved_GBs"],
                     "verified_positions_per_s": var["verified_positions_per_s"]}
    return out


def _row_window(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, Ts=(1, 2, 3, 4, 5, 6), rounds=24,
                warm=8):
    """Kernel cost against the draft window: ReplaySSM verify and the per-draft
    snapshot route for T = 1..6 at one workload's shape, each as a multiple of
    the one-token standard decode step at that shape."""
    wl = synth.WORKLOADS[cfg_id]
    sh = wl.shape
    B, H, D, N, G = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups
    states = [torch.randn((B, H, D, N), device=dev) for _ in range(2)]
    std = _standard_step_row(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, states)
    del states
    out = {"workload": ("Gated DeltaNet" if gdn else "Mamba-2") +
                       f" verify against the draft window, batch {B}, {H} heads, head dim {D}, state {N}, "
                       f"{G} group(s), ring capacity {sh.capacity}; two layer instances rotated; "
                       f"acceptance uniform on 0..T",
           "standard_step": std, "T": []}
    for T in Ts:
        print(f"[bench]   window {'gdn' if gdn else 'mamba2'} T={T}", file=sys.stderr, flush=True)
        rv = _row_verify(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, rounds=rounds, warm=warm, T=T,
                         with_standard=False)
        sn = _snapshot_rounds(torch, np, rd, synth, traffic, dev, stream, cfg_id, gdn, T, rounds, warm)
        out["T"].append({
            "T": T, "replay_verify_us": rv["verify_us"], "replay_rollback_us": rv["rollback_us"],
            "replay_commit_verify_us": rv["commit_verify"]["us_per_round"],
            "replay_GBs": rv["achieved_GBs"], "replay_flush_rate": rv["flush_rate"],
            "snapshot_verify_us": sn["verify_us"], "snapshot_commit_us": sn["commit_us"],
            "snapshot_GBs": sn["achieved_GBs"],
            "replay_alg_bytes_avg_all_launches": rv["alg_bytes_avg_all_launches"],
            "replay_launches": rv["launches"],
            "snapshot_alg_bytes": sn["alg_bytes_per_round"], "snapshot_launches": sn["launches"],
            "replay_x_standard": round(rv["verify_us"] / std["us"], 3),
            "snapshot_x_standard": round(sn["verify_us"] / std["us"], 3),
            "speedup": round(sn["verify_us"] / rv["verify_us"], 3)})
    return out


def _row_sweep(torch, np, rd, synth, traffic, dev, stream, capacities=(4, 8, 16, 32)):
    """Append-decode at every ring capacity of the large-layer workload, flush
    and non-flush steps reported separately (an event pair per launch), the
    average over whole ring cycles from HIP-graph replays as well, plus the
    standard step."""
    wl = synth.WORKLOADS[3]
    base, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G = base.batch, base.nheads, base.head_dim, base.state_dim, base.ngroups
    NLs, P = 2, 4

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    gen = torch.Generator(device=dev)
    S0s, params = [], []
    for l in range(NLs):
        gen.manual_seed(seed * 100 + l)
        S0s.append(torch.randn((B, H, D, N), generator=gen, device=dev) * math.sqrt(0.1))
        A, bias = synth.mamba2_head_params(base, seed, 3, layer=l)
        params.append((torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)))
    pool = []
    for p in range(P):
        st = synth.mamba2_step_inputs(base, seed, 3, p)
        pool.append({"v": bf(st["v"]), "k": bf(st["k"]), "q": bf(st["q"]),
                     "dt": torch.from_numpy(st["dt"]).to(dev)})
    y = torch.empty((B, H, D), device=dev)
    res = {"workload": f"Mamba-2 append-decode, batch {B}, {H} heads, head dim {D}, state {N}, "
                       f"{G} groups; two layer instances rotated", "kernel": "replay_append_decode"}
    for L in capacities:
        dims = rd.Dims(B, H, D, N, G, L)
        rings = [rd.Ring(dims, device=dev) for _ in range(NLs)]
        calls = [[rd.prepare_replay_append_decode(dims, S0s[l], rings[l], pool[p]["v"], pool[p]["k"],
                                                  pool[p]["q"], pool[p]["dt"], params[l][1],
                                                  params[l][0], y, stream=stream)
                  for p in range(P)] for l in range(NLs)]
        warm, K = NLs * L, NLs * L * max(2, 64 // L)
        for t in range(warm):
            calls[t % NLs][(t // NLs) % P]()
        ev = _events(torch, K)
        torch.cuda.synchronize()
        for i in range(K):
            t = warm + i
            ev[i][0].record(stream)
            calls[t % NLs][(t // NLs) % P]()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = np.array([1e3 * a_.elapsed_time(b_) for a_, b_ in ev])
        h = np.array([((warm + i) // NLs) % L for i in range(K)])
        fl = h == L - 1
        byts = np.array([traffic.replay_append(B, H, D, N, G, int(x), bool(x == L - 1)) for x in h])
        nf, f = ~fl, fl
        res[f"L{L}"] = {
            "nonflush_us": round(float(us[nf].mean()), 3),
            "nonflush_GBs": round(float(byts[nf].sum() / (us[nf].sum() * 1e-6) / 1e9), 1),
            "nonflush_bytes_per_step": round(float(byts[nf].mean())),
            "flush_us": round(float(us[f].mean()), 3),
            "flush_GBs": round(float(byts[f].sum() / (us[f].sum() * 1e-6) / 1e9), 1),
            "flush_bytes_per_step": round(float(byts[f].mean())),
            "avg_us": round(float(us.mean()), 3),
            "avg_GBs": round(float(byts.sum() / (us.sum() * 1e-6) / 1e9), 1),
            "tokens_per_s": round(float(B / (us.mean() * 1e-6)), 1), "steps_timed": K}
        if ROW_GRAPHS:
            # the graph timing protocol: lcm(L, 16) steps of both layers (whole ring
            # cycles, flushes included) captured once, 5 untimed and 20 timed replays
            steps = NLs * (L * 16 // math.gcd(L, 16))
            t0 = warm + K
            for t in range(t0, t0 + (-t0) % (NLs * L)):   # start the graph on a cycle boundary
                calls[t % NLs][(t // NLs) % P]()
            t0 += (-t0) % (NLs * L)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for t in range(t0, t0 + steps):
                    calls[t % NLs][(t // NLs) % P]()
            ev_g = _events(torch, 20)
            with torch.cuda.stream(stream):
                torch.cuda.synchronize()
                for _ in range(5):
                    graph.replay()
                for i in range(20):
                    ev_g[i][0].record(stream)
                    graph.replay()
                    ev_g[i][1].record(stream)
            torch.cuda.synchronize()
            g_us = sorted(1e3 * a_.elapsed_time(b_) / steps for a_, b_ in ev_g)
            cyc_bytes = float(np.mean([traffic.replay_append(B, H, D, N, G, x, x == L - 1) for x in range(L)]))
            res[f"L{L}"]["graph"] = {"steps_per_replay": steps, "replays_timed": 20, "warmup_replays": 5,
                                     "us_per_step_median": round(g_us[10], 3), "us_per_step_min": round(g_us[0], 3),
                                     "GBs": round(cyc_bytes / (g_us[10] * 1e-6) / 1e9, 1),
                                     "tokens_per_s": round(B / (g_us[10] * 1e-6), 1)}
        errs = [int(r.err.item()) for r in rings]
        if any(errs):
            raise RuntimeError(f"ring anomaly bits set: {errs}")
        del rings, calls
    dims = rd.Dims(B, H, D, N, G, 16)
    std = [[rd.prepare_ssm_decode_step(dims, S0s[l], pool[p]["v"], pool[p]["k"], pool[p]["q"],
                                       pool[p]["dt"], params[l][1], params[l][0], y, stream=stream)
            for p in range(P)] for l in range(NLs)]
    for t in range(8):
        std[t % NLs][(t // NLs) % P]()
    ev = _events(torch, 32)
    torch.cuda.synchronize()
    for i in range(32):
        ev[i][0].record(stream)
        std[i % NLs][(i // NLs) % P]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    su = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in ev]))
    sb = traffic.standard_step(B, H, D, N, G)
    res["standard_step"] = {"kernel": "ssm_decode_step", "us": round(su, 3),
                            "GBs": round(sb / (su * 1e-6) / 1e9, 1), "tokens_per_s": round(B / (su * 1e-6), 1)}
    return res


def _row_gdn_append(torch, np, rd, synth, traffic, dev, stream, n=None):
    """GDN standard decode through the ring (gdn_replay_append_decode) at the GDN
    workload's shape (state size n if given), flush and non-flush steps reported
    separately, against the standard GDN step; two layer instances rotated."""
    wl = synth.WORKLOADS[4]
    sh, seed = wl.shape.with_(T=1), wl.cfg_seed
    if n is not None:
        sh = sh.with_(state_dim=n)
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    NLs, P = 2, 4
    dims = rd.Dims(B, H, D, N, G, L)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    gen = torch.Generator(device=dev)
    S0s = []
    for l in range(NLs):
        gen.manual_seed(seed * 100 + l)
        S0s.append(torch.randn((B, H, D, N), generator=gen, device=dev) * math.sqrt(0.1))
    ins = []
    for p_ in range(P):
        st = synth.gdn_round_inputs(sh, seed, 4, p_)
        ins.append({k_: (bf(v_[:, 0]) if v_.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(v_[:, 0])).to(dev))
                    for k_, v_ in st.items()})
    rings = [rd.Ring(dims, gdn=True, device=dev) for _ in range(NLs)]
    y = torch.empty((B, H, D), device=dev)

    def call(t):
        ip = ins[(t // NLs) % P]
        rd.gdn_replay_append_decode(dims, S0s[t % NLs], rings[t % NLs], ip["v"], ip["k"], ip["q"], ip["g"],
                                    ip["beta"], y, stream=stream)
    warm, K = NLs * L, NLs * L * 4
    for t in range(warm):
        call(t)
    ev = _events(torch, K)
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        call(warm + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    if any(int(r_.err.item()) for r_ in rings):
        raise RuntimeError("ring anomaly bits set in the GDN append row")
    us = np.array([1e3 * a_.elapsed_time(b_) for a_, b_ in ev])
    h = np.array([((warm + i) // NLs) % L for i in range(K)])
    fl = h == L - 1
    byts = np.array([traffic.gdn_append(B, H, D, N, G, int(x), bool(x == L - 1)) for x in h])
    every = [traffic.gdn_append(B, H, D, N, G, (t // NLs) % L, (t // NLs) % L == L - 1) for t in range(warm + K)]
    std = _standard_step_row(torch, np, rd, synth, traffic, dev, stream, 4, True, S0s, shape=sh)
    return {"workload": f"Gated DeltaNet append-decode (flush when full), batch {B}, {H} heads, head dim {D}, "
                        f"state {N}, {G} groups, ring capacity {L}; two layer instances rotated",
            "kernel": "gdn_replay_append_decode", "steps_timed": K,
            "nonflush_us": round(float(us[~fl].mean()), 3),
            "nonflush_GBs": round(float(byts[~fl].sum() / (us[~fl].sum() * 1e-6) / 1e9), 1),
            "flush_us": round(float(us[fl].mean()), 3),
            "flush_GBs": round(float(byts[fl].sum() / (us[fl].sum() * 1e-6) / 1e9), 1),
            "avg_us": round(float(us.mean()), 3),
            "avg_GBs": round(float(byts.sum() / (us.sum() * 1e-6) / 1e9), 1),
            "tokens_per_s": round(float(B / (us.mean() * 1e-6)), 1),
            "alg_bytes_avg_all_launches": round(float(np.mean(every))), "launches": warm + K,
            "standard_step": std, "speedup": round(std["us"] / float(us.mean()), 3)}


def _row_gdn_state_sizes(torch, np, rd, synth, traffic, dev, stream):
    """GDN append-decode at the GDN workload's shape with state size n = 64, 128
    and 256, each against the standard GDN step at the same n."""
    res = {"workload": "Gated DeltaNet append-decode (flush when full), batch 256, 32 heads, head dim 128, "
                       "32 groups, ring capacity 16, state size n in (64, 128, 256); two layer instances rotated",
           "kernel": "gdn_replay_append_decode"}
    for n in (64, 128, 256):
        r = _row_gdn_append(torch, np, rd, synth, traffic, dev, stream, n=n)
        res[f"n{n}"] = {k_: r[k_] for k_ in ("nonflush_us", "flush_us", "avg_us", "avg_GBs", "tokens_per_s",
                                             "speedup")}
        res[f"n{n}"]["frac_of_peak"] = round(r["avg_GBs"] / HBM_PEAK_GBS, 4)
        res[f"n{n}"]["standard_step_us"] = r["standard_step"]["us"]
    return res


def _row_verify_shapes(torch, np, rd, synth, traffic, dev, stream, rounds=24, warm=8):
    """The speculative verify rows (T = 4, L = 16) at other head dims and state
    sizes, the batch scaled so that every shape reads the same 512 MiB of
    checkpoint per round: verify rounds only, two layer instances rotated."""
    res = {"workload": "speculative verify, T=4, ring capacity 16, 32 heads, at head dim d and state size n "
                       "(Mamba-2 with one group, Gated DeltaNet with one group per head), batch chosen so that "
                       "B*32*d*n*4 bytes = 512 MiB; verify rounds only"}
    cases = ((False, 2, 64, 64), (False, 2, 64, 128), (False, 2, 64, 256), (False, 2, 128, 128),
             (False, 2, 128, 256), (True, 4, 128, 64), (True, 4, 64, 128), (True, 4, 128, 128),
             (True, 4, 128, 256))
    for gdn, cfg, d, n in cases:
        B = (512 * 64 * 128) // (d * n)
        print(f"[bench]   verify {'gdn' if gdn else 'mamba2'} d={d} n={n} B={B}", file=sys.stderr, flush=True)
        res[f"{'gdn' if gdn else 'mamba2'}_d{d}_n{n}"] = _row_verify(
            torch, np, rd, synth, traffic, dev, stream, cfg, gdn, rounds=rounds, warm=warm,
            shape={"batch": B, "head_dim": d, "state_dim": n}, light=True)
    return res


def _row_fused_conv(torch, np, rd, synth, traffic, dev, stream):
    """The layer's front-end fused into the append: conv1d + SiLU over the xBC
    channels (C = H d + 2 G n = 4096 at the Nemotron-H-like shape) producing v, k, q
    in the same launch, against the conv kernel followed by the append kernel (its
    v, k, q already in bf16: the cast between them is not counted); two layer
    instances rotated, per-step HIP-event times of eager launches and, under
    `graph`, the median over replays of the same steps captured in HIP graphs."""
    wl = synth.WORKLOADS[1]
    sh, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    C, NLs, K = H * D + 2 * G * N, 2, 8 * L
    dims = rd.Dims(B, H, D, N, G, L)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    st = synth.mamba2_step_inputs(sh, seed, 1, 0)
    ip = {k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(v_).to(dev)) for k_, v_ in st.items()}
    A, bias = synth.mamba2_head_params(sh, seed, 1)
    A, bias = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
    cs_bits, w_bits = synth.conv_layer(B, C, 4, seed, 1)
    w = bf(w_bits)
    x = bf(synth.conv_step_input(B, C, seed, 1, 0))
    y = torch.empty((B, H, D), device=dev)
    conv_out = torch.empty((B, C), device=dev)
    layers = [{"S0": torch.randn((B, H, D, N), device=dev) * math.sqrt(0.1), "ring": rd.Ring(dims, device=dev),
               "cs": [bf(cs_bits), bf(cs_bits)]} for _ in range(NLs)]

    def fused(t):
        Ly = layers[t % NLs]
        rd.replay_append_decode_conv(dims, Ly["S0"], Ly["ring"], Ly["cs"][(t // NLs) % 2], Ly["cs"][(t // NLs + 1) % 2],
                                     x, w, ip["dt"], bias, A, y, stream=stream)

    def unfused(t):
        Ly = layers[t % NLs]
        rd.causal_conv1d_update(Ly["cs"][0], x, w, conv_out, stream=stream)
        rd.replay_append_decode(dims, Ly["S0"], Ly["ring"], ip["v"], ip["k"], ip["q"], ip["dt"], bias, A, y,
                                stream=stream)
    res = {"workload": f"Mamba-2 layer step, batch {B}, {H} heads, head dim {D}, state {N}, {G} groups, "
                       f"ring capacity {L}, conv over C = {C} xBC channels (width 4); two layer instances rotated",
           "kernel": "replay_append_decode_conv", "steps_timed": K}
    byts = float(np.mean([traffic.replay_append_conv(B, H, D, N, G, h, h == L - 1) for h in range(L)]))
    for name, fn in (("unfused_conv_then_append", unfused), ("fused", fused)):
        for Ly in layers:
            rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
        for t in range(NLs * L):
            fn(t)
        ev = _events(torch, K)
        torch.cuda.synchronize()
        for i in range(K):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in ev]))
        res[name] = {"us_per_step": round(us, 3), "GBs": round(byts / (us * 1e-6) / 1e9, 1),
                     "tokens_per_s": round(B / (us * 1e-6), 1)}
    res["alg_bytes_per_step"] = round(byts)
    res["speedup"] = round(res["unfused_conv_then_append"]["us_per_step"] / res["fused"]["us_per_step"], 3)
    # the same two step sequences captured in HIP graphs (one ring cycle of both
    # layers per graph), no launch gaps or per-step events: 5 untimed replays,
    # then 12 timed ones, median
    if ROW_GRAPHS:
        graphs = {}
        for name, fn in (("unfused_conv_then_append", unfused), ("fused", fused)):
            for Ly in layers:
                rd.rssm_ring_reset(dims, Ly["ring"], stream=stream)
            for t in range(NLs * L):
                fn(t)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(NLs * L):
                    fn(t)
            graphs[name] = g
        reps = {name: [] for name in graphs}
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            for _ in range(5):
                for g in graphs.values():
                    g.replay()
            for _ in range(12):
                for name, g in graphs.items():
                    a_, b_ = _events(torch, 1)[0]
                    a_.record(stream)
                    g.replay()
                    b_.record(stream)
                    reps[name].append((a_, b_))
        torch.cuda.synchronize()
        gr = {}
        for name, evs in reps.items():
            us = sorted(1e3 * a_.elapsed_time(b_) / (NLs * L) for a_, b_ in evs)
            gr[name] = {"us_per_step": round(us[len(us) // 2], 3), "GBs": round(byts / (us[len(us) // 2] * 1e-6) / 1e9, 1)}
        gr["speedup"] = round(gr["unfused_conv_then_append"]["us_per_step"] / gr["fused"]["us_per_step"], 3)
        res["graph"] = gr
    return res


def _row_staggered(torch, np, rd, synth, traffic, dev, stream):
    """The headline append-decode with the requests' ring fill levels staggered
    (request b starts with b mod L entries cached, as under continuous batching),
    so that every launch folds about B / L requests instead of every L-th launch
    folding all of them; against the same launches with synchronised rings.  Four
    layer instances rotated, the same algorithmic bytes per launch on average in
    both (every fill level equally often), back-to-back launches timed as one."""
    wl = synth.WORKLOADS[1]
    sh, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    NLs, K = 4, 4 * 4 * L
    dims = rd.Dims(B, H, D, N, G, L)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    st = synth.mamba2_step_inputs(sh, seed, 1, 0)
    ip = {k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(v_).to(dev)) for k_, v_ in st.items()}
    A, bias = synth.mamba2_head_params(sh, seed, 1)
    A, bias = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
    y = torch.empty((B, H, D), device=dev)
    byts = sum(traffic.replay_append(B, H, D, N, G, h, h == L - 1) for h in range(L)) / L
    res = {"workload": f"Mamba-2 append-decode, batch {B}, {H} heads, head dim {D}, state {N}, {G} groups, "
                       f"ring capacity {L}; four layer instances rotated",
           "kernel": "replay_append_decode", "steps_timed": K, "alg_bytes_per_step": round(byts)}
    for name, stagger in (("synchronised", False), ("staggered", True)):
        layers = []
        for l in range(NLs):
            S0 = torch.randn((B, H, D, N), device=dev) * math.sqrt(0.1)
            ring = rd.Ring(dims, device=dev)
            if stagger:
                ring.set_pointers(head=[0] * B, count=[b % L for b in range(B)], pending=[0] * B)
            layers.append(rd.prepare_replay_append_decode(dims, S0, ring, ip["v"], ip["k"], ip["q"], ip["dt"],
                                                          bias, A, y, stream=stream))
            layers[-1].keep_alive = (S0, ring)
        for t in range(4 * NLs * L):          # four ring cycles per layer before timing
            layers[t % NLs]()
        a_, b_ = _events(torch, 1)[0]
        torch.cuda.synchronize()
        a_.record(stream)
        for i in range(K):
            layers[i % NLs]()
        b_.record(stream)
        torch.cuda.synchronize()
        errs = [int(Ly.keep_alive[1].err.item()) for Ly in layers]
        if any(errs):
            raise RuntimeError(f"ring anomaly bits set in the staggered row: {errs}")
        us = 1e3 * a_.elapsed_time(b_) / K
        res[name] = {"avg_us": round(us, 3), "avg_GBs": round(byts / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "tokens_per_s": round(B / (us * 1e-6), 1)}
        del layers
    return res


def _row_state_sizes(torch, np, rd, synth, traffic, dev, stream):
    """Append-decode at the Nemotron-H-like shape with state size n = 64, 128 and
    256 (everything else as the headline), and the standard step beside it; four
    layer instances rotated, back-to-back launches timed as one, averaged over
    whole ring cycles."""
    wl = synth.WORKLOADS[1]
    base, seed = wl.shape, wl.cfg_seed
    NLs = 4
    res = {"workload": f"Mamba-2 append-decode, batch {base.batch}, {base.nheads} heads, head dim "
                       f"{base.head_dim}, {base.ngroups} groups, ring capacity {base.capacity}, state size "
                       f"n in (64, 128, 256); four layer instances rotated", "kernel": "replay_append_decode"}

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    for n in (64, 128, 256):
        sh = base.with_(state_dim=n)
        B, H, D, G, L = sh.batch, sh.nheads, sh.head_dim, sh.ngroups, sh.capacity
        dims = rd.Dims(B, H, D, n, G, L)
        st = synth.mamba2_step_inputs(sh, seed, 1, 0)
        ip = {k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(v_).to(dev)) for k_, v_ in st.items()}
        A, bias = synth.mamba2_head_params(sh, seed, 1)
        A, bias = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
        y = torch.empty((B, H, D), device=dev)
        layers, stds = [], []
        for l in range(NLs):
            S0 = torch.randn((B, H, D, n), device=dev) * math.sqrt(0.1)
            ring = rd.Ring(dims, device=dev)
            layers.append(rd.prepare_replay_append_decode(dims, S0, ring, ip["v"], ip["k"], ip["q"], ip["dt"],
                                                          bias, A, y, stream=stream))
            layers[-1].keep_alive = (S0, ring)
        K = 4 * NLs * L
        for t in range(K):
            layers[t % NLs]()
        a_, b_ = _events(torch, 1)[0]
        torch.cuda.synchronize()
        a_.record(stream)
        for i in range(K):
            layers[i % NLs]()
        b_.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * a_.elapsed_time(b_) / K
        byts = sum(traffic.replay_append(B, H, D, n, G, h, h == L - 1) for h in range(L)) / L
        std = _standard_step_row(torch, np, rd, synth, traffic, dev, stream, 1, False,
                                 [Ly.keep_alive[0] for Ly in layers], shape=sh)
        res[f"n{n}"] = {"avg_us": round(us, 3), "avg_GBs": round(byts / (us * 1e-6) / 1e9, 1),
                        "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "tokens_per_s": round(B / (us * 1e-6), 1), "alg_bytes_per_step": round(byts),
                        "standard_step": std, "speedup": round(std["us"] / us, 3)}
        del layers
    return res


def _row_pooled(torch, np, rd, synth, traffic, dev, stream):
    """Append-decode at the Nemotron-H-like shape with the checkpoints and rings in
    a pool of 2B request rows, each call's batch entries scattered over the pool
    by a seeded permutation (serving layout), against the same launches with row
    = batch entry; two layer instances rotated, per-launch HIP-event times."""
    wl = synth.WORKLOADS[1]
    sh, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    rows, NLs, K = 2 * B, 2, 8 * L
    dims = rd.Dims(B, H, D, N, G, L)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    st = synth.mamba2_step_inputs(sh, seed, 1, 0)
    ip = {k_: (bf(v_) if v_.dtype == np.uint16 else torch.from_numpy(v_).to(dev)) for k_, v_ in st.items()}
    A, bias = synth.mamba2_head_params(sh, seed, 1)
    A, bias = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
    y = torch.empty((B, H, D), device=dev)
    perm = np.random.default_rng(seed).permutation(rows)[:B].astype(np.int32)
    res = {"workload": f"Mamba-2 append-decode, batch {B} over a pool of {rows} rows, {H} heads, head dim {D}, "
                       f"state {N}, {G} groups, ring capacity {L}; two layer instances rotated",
           "kernel": "replay_append_decode", "steps_timed": K}
    for name, pooled in (("batch_rows", False), ("pooled", True)):
        layers = []
        for l in range(NLs):
            S0 = torch.randn((rows if pooled else B, H, D, N), device=dev) * math.sqrt(0.1)
            ring = rd.Ring(dims, device=dev, rows=rows if pooled else None)
            if pooled:
                ring.use_slots(torch.from_numpy(perm).to(dev))
            layers.append(rd.prepare_replay_append_decode(dims, S0, ring, ip["v"], ip["k"], ip["q"], ip["dt"],
                                                          bias, A, y, stream=stream))
            layers[-1].keep_alive = (S0, ring)
        for t in range(4 * NLs * L):
            layers[t % NLs]()
        ev = _events(torch, K)
        torch.cuda.synchronize()
        for i in range(K):
            ev[i][0].record(stream)
            layers[i % NLs]()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in ev]))
        byts = float(np.mean([traffic.replay_append(B, H, D, N, G, h, h == L - 1) for h in range(L)]))
        res[name] = {"avg_us": round(us, 3), "avg_GBs": round(byts / (us * 1e-6) / 1e9, 1)}
        del layers
    return res


def _row_capacity(torch, np, rd, synth, dev, budget=288 * 10**9, B_check=64):
    """Decode-state bytes per request and the largest batch one MI355X's HBM holds
    for one SSM layer, per route (standard, per-draft snapshots, ReplaySSM), at
    the two speculative workloads' shapes; the model is checked against the
    device memory that the routes' buffers actually take for a batch of 64."""
    from ssm_recurrent_decode_amd import capacity
    out = {"budget_bytes": budget}
    for name, cid, gdn in (("mamba2", 2, False), ("gdn", 4, True)):
        sh = synth.WORKLOADS[cid].shape
        H, D, N, G, L, T = sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
        tab = capacity.concurrency_table(H, D, N, G, L, T, gdn, budget)
        torch.cuda.synchronize()
        m0 = torch.cuda.memory_allocated(dev)
        pool = torch.empty((B_check, T + 1, H, D, N), device=dev)
        slot = torch.zeros((B_check,), dtype=torch.int32, device=dev)
        m1 = torch.cuda.memory_allocated(dev)
        del pool, slot
        torch.cuda.synchronize()
        m1b = torch.cuda.memory_allocated(dev)
        S0 = torch.empty((B_check, H, D, N), device=dev)
        ring = rd.Ring(rd.Dims(B_check, H, D, N, G, L), gdn=gdn, device=dev)
        m2 = torch.cuda.memory_allocated(dev)
        del S0, ring
        tab["allocated_check"] = {
            "batch": B_check,
            "snapshot_bytes": m1 - m0,
            "snapshot_model": B_check * capacity.bytes_per_request("snapshot", H, D, N, G, L, T, gdn),
            "replay_bytes": m2 - m1b,
            "replay_model": B_check * capacity.bytes_per_request("replay", H, D, N, G, L, T, gdn) + 4}
        tab["shape"] = f"{H} heads, head dim {D}, state {N}, {G} group(s), ring capacity {L}, T={T}"
        out[name] = tab
    return out


def _row_flush(torch, np, rd, synth, traffic, dev, stream, reps=8):
    """Explicit flush of full rings: Mamba-2 at the Nemotron-H shape after L - 1
    appends, GDN at its verify shape after three fully accepted verify rounds
    (c = 3T); each flush launch timed with HIP events."""
    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    out = {}
    # Mamba-2
    wl = synth.WORKLOADS[1]
    sh, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    dims = rd.Dims(B, H, D, N, G, L)
    S0 = torch.randn((B, H, D, N), device=dev) * math.sqrt(0.1)
    ring = rd.Ring(dims, device=dev)
    A, bias = synth.mamba2_head_params(sh, seed, 1)
    A, bias = torch.from_numpy(A).to(dev), torch.from_numpy(bias).to(dev)
    st = synth.mamba2_step_inputs(sh, seed, 1, 0)
    ip = {"v": bf(st["v"]), "k": bf(st["k"]), "q": bf(st["q"]), "dt": torch.from_numpy(st["dt"]).to(dev)}
    y = torch.empty((B, H, D), device=dev)
    app = rd.prepare_replay_append_decode(dims, S0, ring, ip["v"], ip["k"], ip["q"], ip["dt"], bias, A, y,
                                          stream=stream)
    ev = _events(torch, reps)
    for i in range(reps + 1):
        for _ in range(L - 1):
            app()
        if i > 0:
            ev[i - 1][0].record(stream)
        rd.replay_flush(dims, S0, ring, stream=stream)
        if i > 0:
            ev[i - 1][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in ev]))
    byts = traffic.replay_flush(B, H, D, N, G, L - 1)
    out["mamba2"] = {"workload": f"replay_flush of {L - 1} entries, batch {B}, {H} heads, head dim {D}, "
                                 f"state {N}, {G} groups", "us": round(us, 3),
                     "achieved_GBs": round(byts / (us * 1e-6) / 1e9, 1), "alg_bytes": byts,
                     "launches": reps + 1}
    del S0, ring
    # GDN
    wl = synth.WORKLOADS[4]
    sh, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G, L, T = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity, sh.T
    dims = rd.Dims(B, H, D, N, G, L)
    S0 = torch.randn((B, H, D, N), device=dev) * math.sqrt(0.1)
    ring = rd.Ring(dims, gdn=True, device=dev)
    st = synth.gdn_round_inputs(sh, seed, 4, 0)
    ip = {"v": bf(st["v"]), "k": bf(st["k"]), "q": bf(st["q"]), "g": torch.from_numpy(st["g"]).to(dev),
          "beta": torch.from_numpy(st["beta"]).to(dev)}
    y = torch.empty((B, T, H, D), device=dev)
    acc_all = torch.full((B,), T, dtype=torch.int32, device=dev)
    rounds = (L - T) // T           # c = rounds * T committed, no early flush on the way
    ev = _events(torch, reps)
    for i in range(reps + 1):
        for _ in range(rounds):
            rd.gdn_replay_verify_T(dims, T, S0, ring, ip["v"], ip["k"], ip["q"], ip["g"], ip["beta"], y,
                                   stream=stream)
            rd.replay_rollback(dims, ring, acc_all, stream=stream)
        if i > 0:
            ev[i - 1][0].record(stream)
        rd.gdn_replay_flush(dims, S0, ring, stream=stream)
        if i > 0:
            ev[i - 1][1].record(stream)
    torch.cuda.synchronize()
    if int(ring.err.item()) != 0:
        raise RuntimeError("ring anomaly bits set in the flush row")
    us = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in ev]))
    byts = traffic.gdn_flush(B, H, D, N, G, rounds * T)
    # the verify rounds that fill the rings (committed count r T before round r)
    buildup = (reps + 1) * sum(_verify_bytes(traffic, True, H, D, N, G, T, L, np.full(B, r * T))
                               for r in range(rounds))
    out["gdn"] = {"workload": f"gdn_replay_flush of {rounds * T} entries, batch {B}, {H} heads, head dim {D}, "
                              f"state {N}, {G} groups", "us": round(us, 3),
                  "achieved_GBs": round(byts / (us * 1e-6) / 1e9, 1), "alg_bytes": byts,
                  "launches": reps + 1, "buildup_verify_launches": (reps + 1) * rounds,
                  "buildup_verify_alg_bytes_total": int(buildup)}
    return out


def _rows(torch, np, rd, synth, traffic, dev, stream, only=None):
    """Every measured row (or the named subset); a progress line per row goes to
    stderr (stdout keeps the one JSON line)."""
    rows = [
        ("speculative_verify", lambda: _row_verify(torch, np, rd, synth, traffic, dev, stream, 2, False)),
        ("gdn_speculative_verify", lambda: _row_verify(torch, np, rd, synth, traffic, dev, stream, 4, True)),
        # the speculative workload with keys and queries shared by groups of four
        # heads instead of all 32 (a sensitivity run of the group count)
        ("speculative_verify_groups8", lambda: _row_verify(torch, np, rd, synth, traffic, dev, stream, 2, False,
                                                           rounds=32, G=8)),
        ("capacity_sweep", lambda: _row_sweep(torch, np, rd, synth, traffic, dev, stream)),
        ("explicit_flush", lambda: _row_flush(torch, np, rd, synth, traffic, dev, stream)),
        ("gdn_append_decode", lambda: _row_gdn_append(torch, np, rd, synth, traffic, dev, stream)),
        ("max_concurrency", lambda: _row_capacity(torch, np, rd, synth, dev)),
        ("pooled_append_decode", lambda: _row_pooled(torch, np, rd, synth, traffic, dev, stream)),
        ("staggered_append_decode", lambda: _row_staggered(torch, np, rd, synth, traffic, dev, stream)),
        ("state_sizes", lambda: _row_state_sizes(torch, np, rd, synth, traffic, dev, stream)),
        ("gdn_state_sizes", lambda: _row_gdn_state_sizes(torch, np, rd, synth, traffic, dev, stream)),
        ("verify_shapes", lambda: _row_verify_shapes(torch, np, rd, synth, traffic, dev, stream)),
        ("fused_front_end", lambda: _row_fused_conv(torch, np, rd, synth, traffic, dev, stream)),
        ("storage_precision", lambda: _row_precision(torch, np, rd, synth, traffic, dev, stream)),
        ("window_sweep", lambda: {"mamba2": _row_window(torch, np, rd, synth, traffic, dev, stream, 2, False),
                                  "gdn": _row_window(torch, np, rd, synth, traffic, dev, stream, 4, True)}),
    ]
    if only is not None:
        unknown = set(only) - {name for name, _ in rows}
        if unknown:
            raise SystemExit(f"unknown rows: {sorted(unknown)}")
        rows = [(name, fn) for name, fn in rows if name in only]
    out = {}
    failed = None
    for name, fn in rows:
        if failed is not None:   # after a failure the device may be unusable: stop there
            out[name] = {"skipped": f"row {failed} failed"}
            continue
        print(f"[bench] row {name}", file=sys.stderr, flush=True)
        try:
            out[name] = fn()
        except Exception as e:  # recorded in the line (and the traceback on stderr); the headline stays
            traceback.print_exc(file=sys.stderr)
            out[name] = {"error": f"{type(e).__name__}: {e}"}
            failed = name
    return out


def main(argv=None) -> int:
    a = _args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step "
              "(requests shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        return 2

    if a.calibrate_copy:
        _calibrate_copy()
        return 0

    import numpy as np
    import torch

    import ssm_recurrent_decode_amd as rd
    from ssm_recurrent_decode_amd import profiling, synth, traffic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[1]
    sh, seed = wl.shape, wl.cfg_seed
    B, H, D, N, G, L = sh.batch, sh.nheads, sh.head_dim, sh.state_dim, sh.ngroups, sh.capacity
    C, W = wl.conv_channels, wl.conv_width
    NL, P = a.layers, a.pool
    dims = rd.Dims(B, H, D, N, G, L)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- layer instances: checkpoint, ring, per-head params, conv state and taps
    gen = torch.Generator(device=dev)
    layers = []
    for l in range(NL):
        gen.manual_seed(seed * 100 + l)
        S0 = torch.randn((B, H, D, N), generator=gen, device=dev) * math.sqrt(0.1)
        A, bias = synth.mamba2_head_params(sh, seed, 1, layer=l)
        cst, cw = synth.conv_layer(B, C, W, seed, 1, layer=l)
        layers.append({"S0": S0, "ring": rd.Ring(dims, device=dev), "A": torch.from_numpy(A).to(dev),
                       "bias": torch.from_numpy(bias).to(dev), "conv_state": bf(cst), "conv_w": bf(cw)})
    # ---- pool of step inputs (cycled; values do not change the work done)
    pool = []
    for p in range(P):
        st = synth.mamba2_step_inputs(sh, seed, 1, p)
        pool.append({"v": bf(st["v"]), "k": bf(st["k"]), "q": bf(st["q"]),
                     "dt": torch.from_numpy(st["dt"]).to(dev),
                     "x": bf(synth.conv_step_input(B, C, seed, 1, p))})
    y = torch.empty((B, H, D), device=dev)
    conv_out = torch.empty((B, C), device=dev)
    side = torch.cuda.Stream(device=dev)          # default priority
    stream = side

    calls = []
    for l in range(NL):
        Ly = layers[l]
        per = []
        for p in range(P):
            ip = pool[p]
            conv = rd.prepare_causal_conv1d_update(Ly["conv_state"], ip["x"], Ly["conv_w"], conv_out,
                                                   stream=stream)
            app = rd.prepare_replay_append_decode(dims, Ly["S0"], Ly["ring"], ip["v"], ip["k"], ip["q"],
                                                  ip["dt"], Ly["bias"], Ly["A"], y, stream=stream)
            per.append((conv, app))
        calls.append(per)

    def step_calls(t):
        return calls[t % NL][(t // NL) % P]

    # ---- warmup
    torch.cuda.synchronize()
    for t in range(a.warmup):
        conv, app = step_calls(t)
        conv()
        app()
    torch.cuda.synchronize()

    # ring fill level before each timed launch, from the integer schedule of each layer
    def cached_before(step_index):
        layer_step = step_index // NL            # steps this layer has taken before
        return layer_step % L

    K = a.steps
    cyc = NL * L                       # one ring cycle of every rotated layer
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # eager pass: the step as launched (conv, then replay), timed as a whole
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        conv, app = step_calls(a.warmup + i)
        conv()
        app()
    end.record(stream)
    end.synchronize()
    eager_ms = start.elapsed_time(end)
    # the dominant kernel alone over whole ring cycles of every layer, whatever
    # K is: K_kern launches back to back on its stream (a multiple of NL * L, so
    # every layer folds its ring once per cycle and the bytes are the L-cycle
    # average exactly), HIP events around the whole run.  It follows eight
    # untimed cycles and two cycles with an event pair around every launch (the
    # launches that fold the ring and those that do not, separately), all
    # enqueued without a host synchronisation in between: after the GPU idles,
    # even briefly, the first cycles of back-to-back launches run 1-40 % slower
    # on this part (measured 78, 61, 56, 55, 55 and 55 us against 54.4 after).
    K_kern = cyc * max(8, math.ceil(K / cyc))
    t_warm = a.warmup + K
    t_cls = t_warm + 8 * cyc
    n_cls = 2 * cyc
    t_kern = t_cls + n_cls
    ev_cls = _events(torch, n_cls)
    ev_cyc = _events(torch, K_kern // cyc)
    torch.cuda.synchronize()
    for i in range(8 * cyc):
        step_calls(t_warm + i)[1]()
    for i in range(n_cls):
        ev_cls[i][0].record(stream)
        step_calls(t_cls + i)[1]()
        ev_cls[i][1].record(stream)
    start.record(stream)
    for i in range(K_kern):
        if i % cyc == 0:
            ev_cyc[i // cyc][0].record(stream)
        step_calls(t_kern + i)[1]()
        if i % cyc == cyc - 1:
            ev_cyc[i // cyc][1].record(stream)
    end.record(stream)
    end.synchronize()
    kern_avg_ms = start.elapsed_time(end) / K_kern
    cycle_us = [round(1e3 * a_.elapsed_time(b_) / cyc, 3) for a_, b_ in ev_cyc]
    cls_us = {False: [], True: []}
    for i in range(n_cls):
        cls_us[cached_before(t_cls + i) == L - 1].append(1e3 * ev_cls[i][0].elapsed_time(ev_cls[i][1]))
    # the conv1d update alone, back to back (the other kernel of the step)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K_kern):
        step_calls(t_kern + i)[0]()
    end.record(stream)
    end.synchronize()
    conv_avg_ms = start.elapsed_time(end) / K_kern
    graph_info = None
    if not a.no_graph:
        # the step sequence of one ring cycle of every layer (NL * L steps, each
        # conv then append) captured once and replayed: no host launch cost
        # between kernels.  5 untimed replays, then R >= 20 replays each between
        # its own events; the value is taken from the median replay.
        t0 = t_cls + n_cls
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for j in range(cyc):
                conv, app = step_calls(t0 + j)
                conv()
                app()
        R = max(20, math.ceil(K / cyc))
        ev_g = _events(torch, R)
        with torch.cuda.stream(side):
            torch.cuda.synchronize()
            for _ in range(5):            # untimed, and no host synchronisation before the timed ones
                g.replay()
            for i in range(R):
                ev_g[i][0].record(side)
                g.replay()
                ev_g[i][1].record(side)
        torch.cuda.synchronize()
        rep_ms = sorted(a_.elapsed_time(b_) for a_, b_ in ev_g)
        med_ms = rep_ms[R // 2] if R % 2 else 0.5 * (rep_ms[R // 2 - 1] + rep_ms[R // 2])
        step_ms = med_ms / cyc
        graph_info = {"steps_per_replay": cyc, "replays_timed": R, "warmup_replays": 5,
                      "median_ms_per_replay": round(med_ms, 5), "min_ms_per_replay": round(rep_ms[0], 5),
                      "max_ms_per_replay": round(rep_ms[-1], 5),
                      "ms_per_step_median": round(step_ms, 6), "ms_per_step_min": round(rep_ms[0] / cyc, 6),
                      "tokens_per_s_min_replay": round(B * cyc / (rep_ms[0] / 1e3), 1),
                      "steps_timed": R * cyc}
    else:
        step_ms = eager_ms / K
    errs = [int(Ly["ring"].err.item()) for Ly in layers]
    if any(errs):
        raise RuntimeError(f"ring anomaly bits set: {errs}")

    alg_bytes = 0
    nflush = 0
    for i in range(K_kern):
        h = cached_before(t_kern + i)
        fl = (h == L - 1)
        nflush += fl
        alg_bytes += traffic.replay_append(B, H, D, N, G, h, fl)
    achieved = alg_bytes / K_kern / (kern_avg_ms * 1e-3) / 1e9
    b_nf = sum(traffic.replay_append(B, H, D, N, G, h, False) for h in range(L - 1)) / (L - 1)
    b_fl = traffic.replay_append(B, H, D, N, G, L - 1, True)
    nf_us, fl_us = sorted(cls_us[False]), sorted(cls_us[True])
    nf_med, fl_med = nf_us[len(nf_us) // 2], fl_us[len(fl_us) // 2]
    ms_per_step = step_ms
    value = B / (step_ms / 1e3)
    traffic_bytes, traffic_note = profiling.stored_traffic("replay_append_decode")
    ceiling = _ceiling_probes(torch, rd, dev, stream, B * H * D * N * 4)

    out = {
        "metric": "SSM decode tokens/s at batch 256 (Mamba-2 shape); achieved HBM GB/s vs peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "Nemotron-H-like SSM layer decode step: causal conv1d update (3072x3 "
                               "bf16, width 4) + ReplaySSM append-decode, batch 256, 32 heads, "
                               "head dim 64, state 128, 8 groups, ring capacity 16",
                   "batch": B, "nheads": H, "head_dim": D, "state_dim": N, "ngroups": G,
                   "capacity": L, "conv_channels": C, "layer_instances_rotated": NL,
                   "flush_steps_timed": nflush},
        "roofline": {"bound": "hbm", "kernel": "replay_append_decode",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_bytes,
                     "traffic_note": traffic_note,
                     "kernel_avg_us": round(1e3 * kern_avg_ms, 3),
                     "launches_timed": K_kern, "flush_launches_timed": nflush,
                     "cycle_avg_us": cycle_us,
                     "alg_bytes_per_launch": round(alg_bytes / K_kern),
                     "nonflush_launch": {"median_us": round(nf_med, 3), "min_us": round(nf_us[0], 3),
                                         "alg_bytes_avg": round(b_nf),
                                         "achieved_GBs": round(b_nf / (nf_med * 1e-6) / 1e9, 1),
                                         "launches": len(nf_us)},
                     "flush_launch": {"median_us": round(fl_med, 3), "min_us": round(fl_us[0], 3),
                                      "alg_bytes": b_fl,
                                      "achieved_GBs": round(b_fl / (fl_med * 1e-6) / 1e9, 1),
                                      "launches": len(fl_us)},
                     "frac_of_read_probe": round(achieved / ceiling["read_one_launch"]["GBs"], 4)},
        "ceiling_probes": ceiling,
        "conv1d": {"kernel": "causal_conv1d_update", "us": round(1e3 * conv_avg_ms, 3),
                   "achieved_GBs": round(traffic.conv1d(B, C, W) / (conv_avg_ms * 1e-3) / 1e9, 1),
                   "alg_bytes": traffic.conv1d(B, C, W)},
        "timing": {"step": "median of the timed HIP graph replays" if graph_info else "eager launches",
                   "eager_ms_per_step": round(eager_ms / K, 5), "graph": graph_info,
                   "kernel": "HIP events around the back-to-back replay_append_decode launches of "
                             "whole ring cycles of every layer on their stream (launches_timed); "
                             "flush and non-flush launches from a second pass, one event pair each"},
    }

    if not a.no_standard:
        # comparator: the baseline that writes the state back every step
        std_calls = []
        for l in range(NL):
            Ly = layers[l]
            std_calls.append([rd.prepare_ssm_decode_step(dims, Ly["S0"], pool[p]["v"], pool[p]["k"],
                                                         pool[p]["q"], pool[p]["dt"], Ly["bias"],
                                                         Ly["A"], y, stream=stream) for p in range(P)])
        for t in range(32):
            std_calls[t % NL][(t // NL) % P]()
        s_a = torch.cuda.Event(enable_timing=True)
        s_b = torch.cuda.Event(enable_timing=True)
        Ks = max(cyc, min(K, 512))
        torch.cuda.synchronize()
        s_a.record(stream)
        for t in range(Ks):
            std_calls[t % NL][(t // NL) % P]()
        s_b.record(stream)
        s_b.synchronize()
        std_us = 1e3 * s_a.elapsed_time(s_b) / Ks
        std_bytes = traffic.standard_step(B, H, D, N, G)
        out["standard_step"] = {"kernel": "ssm_decode_step", "us_per_step": round(std_us, 3),
                                "achieved_GBs": round(std_bytes / (std_us * 1e-6) / 1e9, 1),
                                "alg_bytes": std_bytes,
                                "replay_speedup": round(std_us / (1e3 * kern_avg_ms), 3)}

    global ROW_GRAPHS
    ROW_GRAPHS = not a.no_graph
    if not a.no_rows:
        del calls, layers
        torch.cuda.empty_cache()
        with torch.cuda.stream(stream):       # the rows' own tensor fills on the kernels' stream
            out["rows"] = _rows(torch, np, rd, synth, traffic, dev, stream,
                                None if a.rows is None else [x for x in a.rows.split(",") if x])

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(a.cpu_steps)
        out["cpu_baseline_all_cores"] = _cpu_baseline_all_cores(a.cpu_steps)
        rows = out.get("rows", {})
        for name, cfg_id, nreq in (("speculative_verify", 2, 512), ("gdn_speculative_verify", 4, 128)):
            if name in rows:
                print(f"[bench] cpu oracle for {name}", file=sys.stderr, flush=True)
                rows[name]["cpu_baseline"] = _cpu_spec_baseline(cfg_id, nreq)
        if "capacity_sweep" in rows:
            print("[bench] cpu oracle for capacity_sweep", file=sys.stderr, flush=True)
            rows["capacity_sweep"]["cpu_baseline"] = _cpu_standard_baseline(3, 96)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
