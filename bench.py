#!/usr/bin/env python3
"""Throughput bench of Sketch Attention compression (libsa on one MI355X).

One step = one sa_compress call over the whole synthetic batch (query prep,
pass 1 per-token logsumexp, pass 2 allocations + sums, finalize), inputs
already resident in HBM.  Prints ONE JSON line.

Default workload: 40 users x 100,000 history tokens, k = 1024 prototypes,
d = 128, bf16 inputs -- the n = 100K, k = 1K x 128 sketch batched over 40
users.  ``--workload`` selects any named config of ``synth.CONFIGS``.

Timing: W warm-up steps, then K steps bracketed by device synchronisation;
each timed step also records HIP events at the library's phase boundaries on
the same stream, giving the average duration of every kernel phase.  The
roofline object reports the dominant kernel (pass 2) against the fp16/bf16
dense MFMA peak.  The CPU baseline times the fp64 oracle on a bounded sample
of the same workload on the host cores and checks the GPU sketches of that
sample against it.

``--target-attention`` times sa_target_attention (300 users x 300
candidates over 1K x 128 sketches) with an HBM roofline.

``--cache-serving`` runs a serving trace through the sketch cache: per
step one host lookup of 300 requests (120 of them users not cached) and one
fill (gather + one sa_compress + scatter) on a side stream.

``--serving-pipeline`` adds the sketch branch to that trace: per batch the
300 requests (300 candidates each) attend their cached sketches in place,
timed with the misses' fill serial and overlapped on a side stream.

``--data-probe`` runs the default workload's kernels on its seeded history
and on an all-zero history (same shapes and instruction streams) and reports
both pass times: a difference is the data dependence of the clock.

``--mfma-ceiling`` times sa_probe_mfma, a loop of fp16 32x32x16 MFMAs with no
memory traffic, on zero, constant and random operands: the matrix cores'
rate on random data is the practical ceiling the pass kernels are held to.

``--backward`` times one sa_compress_backward call per step instead (the
gradients dH, dP, dWk, dWv for a seeded dS, forward recomputation included)
on the same workload; its roofline object reports the token-major dH kernel
and its CPU baseline times the fp64 gradient oracle.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0
METRIC = "history tokens/s + TFLOP/s (%bf16 MFMA peak), SA n=100K,k=1024,d=128"
DEFAULT_WORKLOAD = "c3lit_r40_n100k_d128_k1024"

# HBM bytes per launch of each bench mode's dominant kernel on that mode's
# workload: rocprofv3 --pmc FETCH_SIZE + WRITE_SIZE (KiB per dispatch), each
# scaled by what the same counter reads for a plain device copy of known size
# (--calibrate-copy).  A figure is valid only for the kernel source it was
# measured on: the sha256 of the kernel's sources is recorded beside it and
# the figure is reported as null once they differ.
COPY_CALIBRATION_BYTES = 1 << 30
TRAFFIC = {
    # 1.0263e9 fetched + 1.0410e9 written (40 x 100K tokens, k = 1024, d = 128)
    "pass1_qres": (2067296585, "cef297ec68d3429cb9ae1a8bf88d374a992be6d9f2e827b7fbc4dba3503423a2",
                   ("sa_pass1q.hip", "sa_layout.h", "sa_device.h")),
    # 1.0508e9 fetched + 0.0597e9 written (same workload)
    "pass2_accum": (1110476800, "2665c3bdef7508bcdfa688c5baa2451edda846c365be005d8835317ad3fd5fef",
                    ("sa_pass2.hip", "sa_layout.h", "sa_device.h")),
    # 1.3163e9 fetched + 2.0680e9 written (same workload, --backward)
    "bwd_dh": (3384286289, "ea506718fbdb3929200410ceb488213ff1c3e8044723a6ea56600202deaf832d",
               ("sa_bwd.hip", "sa_layout.h", "sa_device.h")),
    # 1.8658e8 fetched + 0.4608e8 written (300 users x 300 candidates, --target-attention)
    "ta_attend": (232547216, "7fe0b40aabfc73acab82beed9163ae42dd37fdd3dc7c16f5d114279d1cae1736",
                  ("sa_target.hip", "sa_layout.h", "sa_device.h")),
}


# MFMA busy fraction of a kernel (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8
# x 1024 SIMDs) and the shader clock under that load (GRBM_GUI_ACTIVE / 8 over the
# kernel's time), from rocprofv3 --pmc on the default workload; valid, like the
# traffic figures, only for the kernel sources they were taken on (null after).
COUNTERS = {
    "pass1_qres": ({"mfma_busy": 0.590, "clock_mhz": 1735.0},
                   "cef297ec68d3429cb9ae1a8bf88d374a992be6d9f2e827b7fbc4dba3503423a2",
                   ("sa_pass1q.hip", "sa_layout.h", "sa_device.h")),
    "pass2_accum": ({"mfma_busy": 0.654, "clock_mhz": 1761.0},
                    "2665c3bdef7508bcdfa688c5baa2451edda846c365be005d8835317ad3fd5fef",
                    ("sa_pass2.hip", "sa_layout.h", "sa_device.h")),
}

# The pages' own efficiency figures, context only: analytic FLOP ratios of the
# cached-sketch path against direct target attention over the 100K history, with
# no hardware stated (blog "100,000 videos in your pocket", "The numbers"; review
# page, "Key claims under review").
PAGES_CONTEXT = {
    "training_flop_ratio": 49.9,
    "training_setting": "R = 40 users per batch, cache-hit rate 0.5",
    "serving_flop_ratio": 63.9,
    "serving_setting": "R = 300 requests, cache-hit rate 0.6",
    "note": "analytic FLOP ratios of the cache-hit path vs direct STCA at 100K; not measured, no hardware",
}


def sources_digest(names) -> str:
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "prototype_attention_compression_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counters(kernel: str):
    """Stored counter figures of ``kernel``, or None once its sources changed."""
    if kernel not in COUNTERS:
        return None
    vals, digest, names = COUNTERS[kernel]
    return dict(vals) if sources_digest(names) == digest else None


def executed_mfma_flop(lengths, k: int, d: int, path: str) -> float:
    """MFMA FLOP the kernels execute for one step (not the algorithmic 4 N k d):
    two passes recompute every logit (pass 1: 2 k d per tile-padded token; pass
    2: 4 k d plus the -l step's 2 k 16), the one-pass kernel computes each once
    (4 k d); the query preparation and the value projection add 2 k d^2 and
    3 x 2 R k d^2 (three-term split)."""
    lens = np.asarray(lengths, dtype=np.int64)
    n_pad = float(((lens + 127) // 128 * 128).sum())
    per_token = 4.0 * k * d if path == "one" else 2.0 * k * d + 4.0 * k * d + 2.0 * k * 16
    return n_pad * per_token + 2.0 * k * d * d + 6.0 * len(lens) * k * d * d


def oracle_chunk_one_thread(inp) -> dict:
    """The fp64 oracle on one 8192-token chunk of the workload with one BLAS
    thread (a per-core reference beside the multi-core baseline)."""
    import threadpoolctl

    from oracle import sketch_one

    n = min(8192, int(inp.lengths[0]))
    Hu = inp.H[:n]
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        sketch_one(Hu, inp.Wk, inp.Wv, inp.P)
        t = time.perf_counter() - t0
    return {"tokens": n, "seconds": t, "tokens_per_s": n / t, "threads": 1}


def measured_traffic(kernel: str):
    """Counter-measured HBM bytes per launch of ``kernel``, or None when its
    sources changed since the counters were taken."""
    nbytes, digest, names = TRAFFIC[kernel]
    return nbytes if sources_digest(names) == digest else None


class _Hip:
    """The few HIP runtime calls the bench needs for phase events."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def _upload(inp, torch, dev):
    if inp.dtype == "bf16":
        t = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
        H, Wk, Wv, P = t(inp.H_bits), t(inp.Wk_bits), t(inp.Wv_bits), t(inp.P_bits)
    else:
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        H, Wk, Wv, P = t(inp.H), t(inp.Wk), t(inp.Wv), t(inp.P)
    off = torch.from_numpy(inp.offsets).to(dev)
    mask = None if inp.mask is None else torch.from_numpy(inp.mask).to(dev)
    return H, off, Wk, Wv, P, mask


def cpu_baseline(inp, S_gpu, budget_s: float):
    """fp64 oracle on the host cores over a bounded sample of users."""
    import threadpoolctl

    from oracle import sketch_one

    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(cores):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        users, tokens, t_total = [], 0, 0.0
        errs = []
        for u in range(inp.R):
            sl = inp.user_slice(u)
            Hu = inp.H[sl] if inp.mask is None else inp.H[sl][inp.mask[sl] != 0]
            t0 = time.perf_counter()
            S, _ = sketch_one(Hu, inp.Wk, inp.Wv, inp.P)
            t_total += time.perf_counter() - t0
            users.append(u)
            tokens += Hu.shape[0]
            ref = S
            diff = np.abs(S_gpu[u].astype(np.float64) - ref)
            errs.append((diff.max(), np.abs(ref).max(), diff.sum(), np.abs(ref).sum()))
            if t_total >= budget_s:
                break
    max_rel = max(e[0] for e in errs) / max(max(e[1] for e in errs), 1e-300)
    mean_rel = sum(e[2] for e in errs) / max(sum(e[3] for e in errs), 1e-300)
    return {
        "value": tokens / t_total,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"users {users[0]}..{users[-1]} ({len(users)} of {inp.R}, {tokens} tokens), "
                  f"numpy fp64, {t_total:.1f} s",
        "parity_on_sample": {"max_rel": max_rel, "mean_rel": mean_rel},
    }


def _calibration_copy(torch, dev):
    """One plain device-to-device copy of known size, for counter scaling."""
    src = torch.ones(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline_backward(inp, dS, dH_gpu, budget_s: float):
    """fp64 gradient oracle on the host cores over a bounded sample of users."""
    import threadpoolctl

    from oracle import sketch_one_grad

    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(cores):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        users, tokens, t_total = [], 0, 0.0
        errs = []
        for u in range(inp.R):
            sl = inp.user_slice(u)
            keep = slice(None) if inp.mask is None else (inp.mask[sl] != 0)
            Hu = inp.H[sl][keep]
            t0 = time.perf_counter()
            gH, _, _, _ = sketch_one_grad(Hu, inp.Wk, inp.Wv, inp.P, dS[u])
            t_total += time.perf_counter() - t0
            users.append(u)
            tokens += Hu.shape[0]
            diff = np.abs(dH_gpu[sl][keep].astype(np.float64) - gH)
            errs.append((diff.max(), np.abs(gH).max(), diff.sum(), np.abs(gH).sum()))
            if t_total >= budget_s:
                break
    max_rel = max(e[0] for e in errs) / max(max(e[1] for e in errs), 1e-300)
    mean_rel = sum(e[2] for e in errs) / max(sum(e[3] for e in errs), 1e-300)
    return {
        "value": tokens / t_total,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"users {users[0]}..{users[-1]} ({len(users)} of {inp.R}, {tokens} tokens), "
                  f"numpy fp64 gradients, {t_total:.1f} s",
        "parity_on_sample": {"dH_max_rel": max_rel, "dH_mean_rel": mean_rel},
    }


def bench_backward(args, inp, torch, dev, sa):
    """Times sa_compress_backward (forward recomputation included), or with
    ``--with-sbar`` sa_compress_backward_with_sbar on the forward's Sbar and
    masses (computed once before the timed region, as a training step's
    forward leaves them), plus the forward that writes them, timed apart."""
    from synth import make_sketch_grad

    H, off, Wk, Wv, P, mask = _upload(inp, torch, dev)
    R, N, d, k = inp.R, inp.N, inp.d, inp.k
    n_valid = inp.valid_tokens()
    dS_host = make_sketch_grad(R, k, d, seed=7)
    dS = torch.from_numpy(dS_host).to(dev)
    ws = torch.empty(sa.backward_workspace_size(R, N, d, k), dtype=torch.uint8, device=dev)
    dH = torch.empty((N, d), dtype=torch.float32, device=dev)
    dP = torch.empty((k, d), dtype=torch.float32, device=dev)
    dWk = torch.empty((d, d), dtype=torch.float32, device=dev)
    dWv = torch.empty((d, d), dtype=torch.float32, device=dev)
    hip = _Hip()
    n_ev = sa._lib.NUM_BWD_PHASE_EVENTS
    step_events = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)]
    ev_arrays = [(ctypes.c_void_p * n_ev)(*evs) for evs in step_events]
    pb = sa._lib.problem(R, N, d, k, sa.SA_BF16)
    ptr = sa._lib._ptr
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    fwd_ms = None
    if args.with_sbar:
        S = torch.empty((R, k, d), dtype=torch.float32, device=dev)
        mass = torch.empty((R, k), dtype=torch.float32, device=dev)
        Sbar = torch.empty((R, k, d), dtype=torch.float32, device=dev)

        def fwd():
            st = sa._lib.raw_compress_with_sbar(pb, ptr(H), ptr(off), ptr(mask), ptr(Wk), ptr(Wv), ptr(P), ptr(S),
                                                ptr(mass), ptr(Sbar), ptr(ws), ws.numel(), stream, None)
            if st != sa.SA_OK:
                raise sa.SaError(st, "sa_compress_with_sbar")

        for _ in range(args.warmup):
            fwd()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fwd()
        e1.record()
        torch.cuda.synchronize()
        fwd_ms = e0.elapsed_time(e1) / args.steps

    def step(events=None):
        if args.with_sbar:
            st = sa._lib.raw_compress_backward_with_sbar(pb, ptr(H), ptr(off), ptr(mask), ptr(Wk), ptr(Wv), ptr(P),
                                                         ptr(Sbar), ptr(mass), ptr(dS), ptr(dH), ptr(dP), ptr(dWk),
                                                         ptr(dWv), ptr(ws), ws.numel(), stream, events)
        else:
            st = sa._lib.raw_compress_backward(pb, ptr(H), ptr(off), ptr(mask), ptr(Wk), ptr(Wv), ptr(P), ptr(dS),
                                               ptr(dH), ptr(dP), ptr(dWk), ptr(dWv), ptr(ws), ws.numel(), stream,
                                               events)
        if st != sa.SA_OK:
            raise sa.SaError(st, "sa_compress_backward")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(ev_arrays[i])
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    phases = ["forward_pass1" if args.with_sbar else "forward_recompute", "per_user", "dh", "e", "params"]
    phase_ms = {p: 0.0 for p in phases}
    for evs in step_events:
        for i, p in enumerate(phases):
            phase_ms[p] += hip.elapsed_ms(evs[i], evs[i + 1]) / args.steps
        for e in evs:
            hip.destroy(e)
    nkd = float(n_valid) * k * d
    # algorithmic work of the backward proper: logits and Z.h once (2 x 2nkd),
    # E = dL h (2nkd), dh's two contractions (4nkd)
    algo_flop = 10.0 * nkd
    dh_flop = 8.0 * nkd     # bwd_dh: logits, Z.h and the two contractions of dh
    dh_s = phase_ms["dh"] * 1e-3
    dh_achieved = dh_flop / dh_s / 1e12 if dh_s > 0 else 0.0
    out = {
        "metric": "history tokens/s (backward: dH, dP, dWk, dWv), SA n=100K,k=1024,d=128",
        "value": n_valid / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": inp.name, "users": R, "tokens": n_valid, "k": k, "d": d,
                   "input_dtype": inp.dtype, "parallelism": "single_gpu",
                   "pass": "backward_with_sbar" if args.with_sbar else "backward"},
        "tflops": algo_flop / (ms_step * 1e-3) / 1e12,
        "phase_ms": phase_ms,
        "wall_s_timed": t_wall,
        "roofline": {
            "kernel": "bwd_dh",
            "bound": "mfma",
            "achieved": dh_achieved,
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": dh_achieved / PEAK_MFMA_F16_TFLOPS,
            "traffic": measured_traffic("bwd_dh") if inp.name == DEFAULT_WORKLOAD else None,
            "per_launch_flop": dh_flop,
            "avg_launch_ms": phase_ms["dh"],
        },
    }
    if fwd_ms is not None:
        # the training step's forward (sa_compress_with_sbar) and the sum
        out["forward_with_sbar_ms"] = fwd_ms
        out["train_step_ms"] = fwd_ms + ms_step
    if args.calibrate_copy:
        _calibration_copy(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(inp, dS_host, dH.cpu().numpy(), args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


TA_USERS, TA_CANDIDATES = 300, 300   # serving: ~300 candidates per request against one sketch


def bench_target(args, torch, dev, sa):
    """Times sa_target_attention: 300 users x 300 candidates over 1K x 128
    sketches (the serving reuse operating point), inputs resident in HBM."""
    from synth import make_candidates, make_sketches

    R, C_u, k, d = TA_USERS, TA_CANDIDATES, 1024, 128
    Qf, Qbits, off_h = make_candidates([C_u] * R, d, seed=11)
    S_h = make_sketches(R, k, d, seed=12)
    C = int(off_h[-1])
    Q = torch.from_numpy(Qbits.view(np.int16)).view(torch.bfloat16).to(dev)
    off = torch.from_numpy(off_h).to(dev)
    S = torch.from_numpy(S_h).to(dev)
    out_t = torch.empty((C, d), dtype=torch.float32, device=dev)
    ws = torch.empty(sa.target_attention_workspace_size(R, C, d, k), dtype=torch.uint8, device=dev)

    def step():
        sa.target_attention(Q, off, S, out=out_t, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    flop = 4.0 * C * k * d                       # logits and the weighted sum, once each
    nbytes = 4.0 * R * k * d + 2.0 * C * d + 4.0 * C * d   # sketches once per user, queries, outputs
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "candidates/s (sketch-branch target attention), 1K x 128 sketches",
        "value": C / (ms_step * 1e-3),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"target_r{R}_c{C_u}_d{d}_k{k}", "users": R, "candidates": C, "k": k, "d": d,
                   "parallelism": "single_gpu", "op": "target_attention"},
        "tflops": flop / (ms_step * 1e-3) / 1e12,
        "wall_s_timed": t_wall,
        "roofline": {
            "kernel": "ta_attend",
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": measured_traffic("ta_attend"),
            "per_launch_bytes": nbytes,
            "avg_launch_ms": ms_step,
        },
    }
    if args.calibrate_copy:
        _calibration_copy(torch, dev)
    if not args.no_cpu_baseline:
        import threadpoolctl

        from oracle import target_attention_one
        cores = len(os.sched_getaffinity(0))
        with threadpoolctl.threadpool_limits(cores):
            threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
            n_c, t_total, u = 0, 0.0, 0
            while u < R and t_total < args.cpu_budget:
                lo, hi = int(off_h[u]), int(off_h[u + 1])
                t0 = time.perf_counter()
                target_attention_one(Qf[lo:hi], S_h[u])
                t_total += time.perf_counter() - t0
                n_c += hi - lo
                u += 1
        out["cpu_baseline"] = {"value": n_c / t_total, "unit": "candidates/s", "cores": threads, "kind": "oracle",
                               "sample": f"users 0..{u - 1} ({u} of {R}, {n_c} candidates), numpy fp64, "
                                         f"{t_total:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


def bench_cache(args, torch, dev, sa):
    """Serving trace through the sketch cache: batches of 300 requests of
    which 120 are users not in the cache (the miss fraction 0.4 of the
    serving operating point), compressed by one fill per batch."""
    from synth import make_inputs

    R_req, n_new, k, d = 300, 120, 1024, 128
    R_store = R_req + n_new
    g = np.random.default_rng(3)
    lens = np.clip(np.round(g.lognormal(np.log(30000.0), 0.8, size=R_store)), 1000, 100000).astype(np.int64)
    inp = make_inputs(lens, d=d, k=k, seed=13, name="cache_store")
    H, off, Wk, Wv, P, mask = _upload(inp, torch, dev)
    slab = torch.empty((R_req, k, d), dtype=torch.float32, device=dev)
    mass = torch.empty((R_req, k), dtype=torch.float32, device=dev)
    cache = sa.SketchCache(R_req, k, d, 3600.0, slab, mass)
    # workspace for the largest miss batch of the trace
    worst = int(np.sort(lens)[-n_new:].sum())
    pb = sa._lib.problem(R_store, int(inp.offsets[-1]), d, k, sa.SA_BF16)
    need = ctypes.c_size_t(0)
    sa._lib.load().sa_cache_fill_workspace_size(ctypes.byref(pb), R_req, worst, ctypes.byref(need))
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()

    def batch_users(b):   # a window sliding by n_new users: 180 repeat, 120 new
        return (np.arange(R_req, dtype=np.int64) + n_new * b) % R_store

    b = 0
    slots, mu, ms, st = cache.lookup(batch_users(b), 0.0)   # cold start: all misses
    cache.fill(H, inp.offsets, Wk, Wv, P, mu, ms, workspace=ws, stream=side)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        b += 1
        _, mu, ms, _ = cache.lookup(batch_users(b), float(b))
        cache.fill(H, inp.offsets, Wk, Wv, P, mu, ms, workspace=ws, stream=side)
    torch.cuda.synchronize()
    host_s, gpu_ms, hits, misses, miss_tokens = 0.0, 0.0, 0, 0, 0
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        b += 1
        t0 = time.perf_counter()
        _, mu, ms, st = cache.lookup(batch_users(b), float(b))
        host_s += time.perf_counter() - t0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        cache.fill(H, inp.offsets, Wk, Wv, P, mu, ms, workspace=ws, stream=side)
        e1.record(side)
        e1.synchronize()
        gpu_ms += e0.elapsed_time(e1)
        hits += st["hits"]
        misses += st["misses"]
        miss_tokens += int((inp.offsets[mu + 1] - inp.offsets[mu]).sum())
    t_wall = time.perf_counter() - t_wall
    ms_step = t_wall * 1e3 / args.steps
    out = {
        "metric": "serving batches/s through the sketch cache (300 requests, miss fraction 0.4)",
        "value": args.steps / t_wall,
        "unit": "batches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"cache_serving_r{R_req}_new{n_new}_d{d}_k{k}", "requests": R_req,
                   "store_users": R_store, "k": k, "d": d, "parallelism": "single_gpu", "op": "cache_fill"},
        "hit_rate": hits / max(1, hits + misses),
        "misses_per_batch": misses / args.steps,
        "miss_tokens_per_batch": miss_tokens / args.steps,
        "phase_ms": {"lookup_host": host_s * 1e3 / args.steps, "fill_gpu": gpu_ms / args.steps},
        "miss_tokens_per_s_gpu": miss_tokens / (gpu_ms * 1e-3),
        "roofline": None,
    }
    cache.close()
    print(json.dumps(out), flush=True)
    return 0


def bench_serving_pipeline(args, torch, dev, sa):
    """Serving batches through the cache with the sketch branch: 300 requests
    (300 candidates each), 180 cached users and 120 misses per batch.
    Serial: fill the misses, then attend all requests.  Overlapped ("pipeline
    lift"): the misses' fill on a side stream while the cached requests are
    attended on the main stream, then the missed requests."""
    from synth import make_candidates, make_inputs

    R_req, n_new, k, d, C_u = 300, 120, 1024, 128, 300
    R_store = R_req + n_new
    g = np.random.default_rng(3)
    lens = np.clip(np.round(g.lognormal(np.log(30000.0), 0.8, size=R_store)), 1000, 100000).astype(np.int64)
    inp = make_inputs(lens, d=d, k=k, seed=13, name="cache_store")
    H, off, Wk, Wv, P, mask = _upload(inp, torch, dev)
    slab = torch.empty((R_req, k, d), dtype=torch.float32, device=dev)
    cache = sa.SketchCache(R_req, k, d, 3600.0, slab)
    worst = int(np.sort(lens)[-n_new:].sum())
    pb = sa._lib.problem(R_store, int(inp.offsets[-1]), d, k, sa.SA_BF16)
    need = ctypes.c_size_t(0)
    sa._lib.load().sa_cache_fill_workspace_size(ctypes.byref(pb), R_req, worst, ctypes.byref(need))
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    _, Qbits, coff = make_candidates([C_u] * R_req, d, seed=14)
    Q = torch.from_numpy(Qbits.view(np.int16)).view(torch.bfloat16).to(dev)
    off_all = torch.from_numpy(coff).to(dev)
    n_hit = R_req - n_new
    off_hit = torch.from_numpy(coff[:n_hit + 1]).to(dev)
    off_miss = torch.from_numpy(coff[n_hit:] - coff[n_hit]).to(dev)
    Q_hit, Q_miss = Q[:n_hit * C_u], Q[n_hit * C_u:]
    out = torch.empty((R_req * C_u, d), dtype=torch.float32, device=dev)
    out_hit, out_miss = out[:n_hit * C_u], out[n_hit * C_u:]
    ta_ws = torch.empty(sa.target_attention_workspace_size(R_req, R_req * C_u, d, k), dtype=torch.uint8,
                        device=dev)
    ta_ws2 = torch.empty_like(ta_ws)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def window(b):   # hits first: the 180 users of the previous window, then 120 new ones
        return (np.arange(R_req, dtype=np.int64) + n_new * b) % R_store

    def batch(b, overlapped):
        slots, mu, ms, st = cache.lookup(window(b), float(b))
        rows = torch.from_numpy(slots).to(dev)
        if overlapped:
            side.wait_stream(main)
            cache.fill(H, inp.offsets, Wk, Wv, P, mu, ms, workspace=ws, stream=side)
            ev = torch.cuda.Event()
            ev.record(side)
            sa.target_attention(Q_hit, off_hit, slab, out=out_hit, workspace=ta_ws, sketch_rows=rows[:n_hit])
            main.wait_event(ev)
            sa.target_attention(Q_miss, off_miss, slab, out=out_miss, workspace=ta_ws2, sketch_rows=rows[n_hit:])
        else:
            cache.fill(H, inp.offsets, Wk, Wv, P, mu, ms, workspace=ws, stream=main)
            sa.target_attention(Q, off_all, slab, out=out, workspace=ta_ws, sketch_rows=rows)
        return st

    b = 0
    batch(b, False)   # cold start
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for ov in (False, True):
            b += 1
            batch(b, ov)
    torch.cuda.synchronize()
    t = {False: 0.0, True: 0.0}
    hits = misses = 0
    for _ in range(args.steps):
        for ov in (False, True):
            b += 1
            t0 = time.perf_counter()
            st = batch(b, ov)
            torch.cuda.synchronize()
            t[ov] += time.perf_counter() - t0
            hits += st["hits"]
            misses += st["misses"]
    ms_serial = t[False] * 1e3 / args.steps
    ms_overlap = t[True] * 1e3 / args.steps
    res = {
        "metric": "serving batches/s, cache + sketch-branch attention (300 requests x 300 candidates)",
        "value": 1e3 / ms_overlap,
        "unit": "batches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_overlap,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"serving_pipeline_r{R_req}_new{n_new}_c{C_u}_d{d}_k{k}", "requests": R_req,
                   "candidates_per_request": C_u, "store_users": R_store, "k": k, "d": d,
                   "parallelism": "single_gpu", "op": "cache_fill+target_attention"},
        "hit_rate": hits / max(1, hits + misses),
        "ms_serial": ms_serial,
        "ms_overlapped": ms_overlap,
        "roofline": None,
    }
    cache.close()
    print(json.dumps(res), flush=True)
    return 0


OTHER_CONFIGS = ("c1_fp32_n4096_d64_k64", "c2_n100k_d128_k1024", "c3_r40_ragged_d128_k1024",
                 "c4_r120_lognormal_d128_k1024", "c5_r8_n100k_d128_k256", "c5_r8_n100k_d128_k512",
                 "c5_r8_n100k_d128_k2048", "c5mask_r8_n100k_d128_k1024")


INFINITY_CACHE_BYTES = 256 << 20   # MI355X's last-level (MALL) cache


def measure_config(name: str, torch, dev, sa, steps: int = 10, warmup: int = 3, flush=None) -> dict:
    """A short measurement of one named workload: clean timed steps, then the
    same number with phase events for the pass-2 share.  Those steps run warm:
    a history that fits the Infinity Cache stays there between steps.  When
    it fits and ``flush`` (a device buffer of at least twice the cache) is
    given, the steps are timed once more one by one, each after a write of
    the whole buffer that evicts the cache: ``cold_ms`` (median, min)."""
    from synth import make_config

    inp = make_config(name)
    H, off, Wk, Wv, P, mask = _upload(inp, torch, dev)
    R, N, d, k = inp.R, inp.N, inp.d, inp.k
    dt = sa.SA_BF16 if inp.dtype == "bf16" else sa.SA_F32
    ws = torch.empty(sa.workspace_size(R, N, d, k, dt), dtype=torch.uint8, device=dev)
    S = torch.empty((R, k, d), dtype=torch.float32, device=dev)
    m = torch.empty((R, k), dtype=torch.float32, device=dev)
    hip = _Hip()
    n_ev = sa._lib.NUM_PHASE_EVENTS
    evs = [[hip.event() for _ in range(n_ev)] for _ in range(steps)]
    arrs = [(ctypes.c_void_p * n_ev)(*e) for e in evs]

    def step(events=None):
        sa.compress(H, off, Wk, Wv, P, mask=mask, return_mass=True, out=S, mass_out=m, workspace=ws,
                    events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the clean timing window covers about 20 ms of work (at least `steps`
    # steps), after as many warm-up steps again, so that the launch latency
    # at its ends and the clock's transitions weigh little for small workloads
    a.record()
    step()
    b.record()
    torch.cuda.synchronize()
    clean = int(min(2000, max(steps, math.ceil(20.0 / max(a.elapsed_time(b), 1e-3)))))
    for _ in range(clean):
        step()
    a.record()
    for _ in range(clean):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / clean
    for i in range(steps):
        step(arrs[i])
    torch.cuda.synchronize()
    p2 = sum(hip.elapsed_ms(e[2], e[3]) for e in evs) / steps
    p1 = sum(hip.elapsed_ms(e[1], e[2]) for e in evs) / steps
    h_bytes = H.numel() * H.element_size()
    cold = None
    if flush is not None and h_bytes < INFINITY_CACHE_BYTES:
        times = []
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(steps):
            flush.fill_(float(i))
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        cold = {"median": float(np.median(times)), "min": float(np.min(times)), "reps": steps}
    for e in evs:
        for x in e:
            hip.destroy(x)
    n_valid = inp.valid_tokens()
    algo = 4.0 * n_valid * k * d
    out = {"users": R, "tokens": n_valid, "k": k, "d": d, "dtype": inp.dtype, "ms_per_step": ms, "timed_steps": clean,
           "tokens_per_s": n_valid / (ms * 1e-3), "tflops": algo / (ms * 1e-3) / 1e12,
           "pct_peak": algo / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS if inp.dtype == "bf16" else None,
           "pass1_ms": p1, "pass2_ms": p2,
           "pass2_frac": algo / (p2 * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS if inp.dtype == "bf16" else None,
           "cache": "warm" if h_bytes < INFINITY_CACHE_BYTES else "history larger than the Infinity Cache",
           "cold_ms": cold}
    del H, off, Wk, Wv, P, mask, ws, S, m
    return out


def bench_data_probe(args, torch, dev, sa):
    """The headline workload twice through the same kernels: once on its
    seeded history, once on an all-zero history (a valid input: every logit
    is 0, every allocation 1/k, every sketch 0).  Same shapes, launches and
    instruction streams; only the operand data differ.  A time that depends
    on the data shows a clock set by power, not by issue rates."""
    from synth import make_config

    inp = make_config(DEFAULT_WORKLOAD)
    H, off, Wk, Wv, P, mask = _upload(inp, torch, dev)
    R, N, d, k = inp.R, inp.N, inp.d, inp.k
    ws = torch.empty(sa.workspace_size(R, N, d, k), dtype=torch.uint8, device=dev)
    S = torch.empty((R, k, d), dtype=torch.float32, device=dev)
    m = torch.empty((R, k), dtype=torch.float32, device=dev)
    hip = _Hip()
    n_ev = sa._lib.NUM_PHASE_EVENTS
    res = {}
    for name, hist in (("seeded", H), ("zero", torch.zeros_like(H)), ("seeded_again", H)):
        evs = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)]
        arrs = [(ctypes.c_void_p * n_ev)(*e) for e in evs]
        for _ in range(args.warmup):
            sa.compress(hist, off, Wk, Wv, P, mask=mask, return_mass=True, out=S, mass_out=m, workspace=ws)
        torch.cuda.synchronize()
        for i in range(args.steps):
            sa.compress(hist, off, Wk, Wv, P, mask=mask, return_mass=True, out=S, mass_out=m, workspace=ws,
                        events=arrs[i])
        torch.cuda.synchronize()
        ph = {"pass1_lse": 0.0, "pass2_accum": 0.0}
        for e in evs:
            ph["pass1_lse"] += hip.elapsed_ms(e[1], e[2]) / args.steps
            ph["pass2_accum"] += hip.elapsed_ms(e[2], e[3]) / args.steps
            for x in e:
                hip.destroy(x)
        res[name] = ph
        if name == "zero":
            assert not S.any(), "a zero history gives zero sketches"
    algo = 4.0 * N * k * d
    out = {
        "metric": "pass times on seeded vs all-zero history (same kernels)",
        "value": res["zero"]["pass2_accum"] / res["seeded"]["pass2_accum"],
        "unit": "ratio (zero / seeded pass-2 time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": False,
        "data": "synthetic",
        "config": {"workload": DEFAULT_WORKLOAD, "users": R, "tokens": N, "k": k, "d": d},
        "phase_ms": res,
        "pass2_tflops": {n: algo / (v["pass2_accum"] * 1e-3) / 1e12 for n, v in res.items()},
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_mfma_ceiling(args, torch, dev, sa):
    """The matrix cores' rate on zero, constant and random fp16 operands
    (sa_probe_mfma: no memory traffic, two waves per SIMD, four independent
    accumulator chains per wave), each kind warmed up and then timed over
    ``--steps`` launches with events on the current stream.  The random kind
    runs again at the end to show drift."""
    sink = torch.empty(sa._lib.PROBE_SINK_FLOATS, dtype=torch.float32, device=dev)
    iters = 4096
    res = {}
    for name, kind in (("random", 2), ("constant", 1), ("zeros", 0), ("random_again", 2)):
        for _ in range(max(args.warmup, 20)):
            sa._lib.probe_mfma(kind, iters, sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        flop = 0.0
        for _ in range(args.steps):
            flop += sa._lib.probe_mfma(kind, iters, sink)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        res[name] = {"tflops": flop / (ms * 1e-3) / 1e12, "ms_per_launch": ms / args.steps}
        assert torch.isfinite(sink).all()
    out = {
        "metric": "fp16 MFMA rate (32x32x16, operands in registers, no memory traffic)",
        "value": res["random"]["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": max(args.warmup, 20),
        "higher_is_better": True,
        "data": "synthetic",
        "config": {"workload": "mfma_probe_2048_waves", "iters": iters, "mfma_per_iter": 8,
                   "flop_per_launch": float(sa._lib.PROBE_WAVES) * iters * 8 * 32768},
        "by_operands": res,
        "peak": PEAK_MFMA_F16_TFLOPS,
        "frac_random": res["random"]["tflops"] / PEAK_MFMA_F16_TFLOPS,
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the clock settles over the first ten or so steps of a process (5.3, 3.6,
    # 3.3, 3.2 ... 2.85 ms at the default workload), so the default warm-up
    # covers them
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the short measurements of the other workloads")
    ap.add_argument("--path", choices=["auto", "one", "two"], default="auto",
                    help="kernel path: the library's choice, the one-pass or the two-pass kernels")
    ap.add_argument("--target-attention", action="store_true",
                    help="time sketch-branch target attention (300 users x 300 candidates) instead")
    ap.add_argument("--cache-serving", action="store_true",
                    help="time the cache-miss driver on a serving trace (300 requests, 120 misses per batch)")
    ap.add_argument("--serving-pipeline", action="store_true",
                    help="cache + sketch-branch attention per serving batch, serial vs overlapped fill")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gradients through the sketches) instead")
    ap.add_argument("--with-sbar", action="store_true",
                    help="with --backward: hand the forward's Sbar and masses to the backward "
                         "(sa_compress_backward_with_sbar) instead of recomputing its sums")
    ap.add_argument("--data-probe", action="store_true",
                    help="time the headline workload on its seeded history and on an all-zero history")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="time a loop of fp16 MFMAs (no memory traffic) on zero, constant and random operands")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy 1 GiB device-to-device once (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Sketch Attention path here runs on a single "
              "MI355X (users shard across GPUs with no exchange; no multi-GPU run is built). "
              "Use --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import prototype_attention_compression_amd as sa
    from synth import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.target_attention:
        return bench_target(args, torch, dev, sa)
    if args.cache_serving:
        return bench_cache(args, torch, dev, sa)
    if args.serving_pipeline:
        return bench_serving_pipeline(args, torch, dev, sa)
    if args.data_probe:
        return bench_data_probe(args, torch, dev, sa)
    if args.mfma_ceiling:
        return bench_mfma_ceiling(args, torch, dev, sa)
    inp = make_config(args.workload)
    if args.backward:
        return bench_backward(args, inp, torch, dev, sa)
    H, off, Wk, Wv, P, mask = _upload(inp, torch, dev)
    R, N, d, k = inp.R, inp.N, inp.d, inp.k
    n_valid = inp.valid_tokens()
    ws = torch.empty(sa.workspace_size(R, N, d, k, sa.SA_BF16 if inp.dtype == "bf16" else sa.SA_F32),
                     dtype=torch.uint8, device=dev)
    S = torch.empty((R, k, d), dtype=torch.float32, device=dev)
    m = torch.empty((R, k), dtype=torch.float32, device=dev)

    hip = _Hip()
    n_ev = sa._lib.NUM_PHASE_EVENTS
    step_events = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)]
    ev_arrays = [(ctypes.c_void_p * n_ev)(*evs) for evs in step_events]

    def step(events=None):
        sa.compress(H, off, Wk, Wv, P, mask=mask, return_mass=True, out=S, mass_out=m,
                    workspace=ws, events=events, path=args.path)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps carry no phase events (each event record costs a few
    # microseconds between kernels, which shows at small workloads)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    # then the same number of steps again with events at the phase
    # boundaries, for the per-phase durations and the per-step spread
    for i in range(args.steps):
        step(ev_arrays[i])
    torch.cuda.synchronize()

    phases = ["prep", "pass1_lse", "pass2_accum", "finalize"]
    phase_ms = {p: 0.0 for p in phases}
    per_step = []
    for evs in step_events:
        for i, p in enumerate(phases):
            phase_ms[p] += hip.elapsed_ms(evs[i], evs[i + 1]) / args.steps
        per_step.append(hip.elapsed_ms(evs[0], evs[-1]))
    for evs in step_events:
        for e in evs:
            hip.destroy(e)

    algo_flop = 4.0 * n_valid * k * d          # logits + A^T V contractions
    tflops = algo_flop / (ms_step * 1e-3) / 1e12
    tokens_per_s = n_valid / (ms_step * 1e-3)
    p2_s = phase_ms["pass2_accum"] * 1e-3
    p2_achieved = algo_flop / p2_s / 1e12 if p2_s > 0 else 0.0
    path = "two" if args.path == "auto" else args.path
    exec_flop = executed_mfma_flop(inp.lengths, k, d, path) if inp.dtype == "bf16" else None
    two_pass_default = inp.name == DEFAULT_WORKLOAD and args.path != "one"
    traffic = measured_traffic("pass2_accum") if two_pass_default else None
    counters = measured_counters("pass2_accum") if two_pass_default else None
    props = torch.cuda.get_device_properties(dev)
    roofline = {
        "kernel": "pass2_accum",
        "bound": "mfma",
        "achieved": p2_achieved,
        "peak": PEAK_MFMA_F16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": p2_achieved / PEAK_MFMA_F16_TFLOPS,
        # counters were taken on the default workload's two-pass kernels
        "traffic": traffic,
        "per_launch_flop": algo_flop,
        "avg_launch_ms": phase_ms["pass2_accum"],
        # the whole step (every kernel) against the same peak
        "step_frac": tflops / PEAK_MFMA_F16_TFLOPS,
        "mfma_busy": None if counters is None else counters["mfma_busy"],
        "hbm_gbps": None if traffic is None or p2_s <= 0 else traffic / p2_s / 1e9,
    }
    # the second kernel of the step: pass 1's logit contraction (2 N k d
    # algorithmic FLOP) and its H read + fp16 copy write
    p1_s = phase_ms["pass1_lse"] * 1e-3
    p1_flop = 2.0 * n_valid * k * d
    p1_traffic = measured_traffic("pass1_qres") if two_pass_default else None
    p1_counters = measured_counters("pass1_qres") if two_pass_default else None
    if path == "two" and p1_s > 0:
        roofline["pass1"] = {
            "kernel": "pass1_qres",
            "bound": "mfma",
            "achieved": p1_flop / p1_s / 1e12,
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": p1_flop / p1_s / 1e12 / PEAK_MFMA_F16_TFLOPS,
            "avg_launch_ms": phase_ms["pass1_lse"],
            "traffic": p1_traffic,
            "hbm_gbps": None if p1_traffic is None else p1_traffic / p1_s / 1e9,
            "mfma_busy": None if p1_counters is None else p1_counters["mfma_busy"],
        }
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if inp.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": inp.name, "users": R, "tokens": n_valid, "k": k, "d": d,
                   "input_dtype": inp.dtype, "parallelism": "single_gpu"},
        "tflops": tflops,
        "pct_peak": tflops / PEAK_MFMA_F16_TFLOPS,
        "exec_tflops": None if exec_flop is None else exec_flop / (ms_step * 1e-3) / 1e12,
        # spread over the steps that carry phase events
        "step_ms": {"median": float(np.median(per_step)), "min": float(np.min(per_step)), "reps": len(per_step)},
        "phase_ms": phase_ms,
        "wall_s_timed": t_wall,
        "roofline": roofline,
        "gpu": {"name": props.name, "cus": props.multi_processor_count,
                "clock_max_mhz": getattr(props, "clock_rate", 0) / 1000.0 or None,
                "clock_under_load_mhz": None if counters is None else counters["clock_mhz"],
                "rocm": torch.version.hip},
        "seed": int(inp.seed),
        "pages_context": PAGES_CONTEXT,
    }
    if args.calibrate_copy:
        _calibration_copy(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, S.cpu().numpy(), args.cpu_budget)
        out["cpu_baseline"]["one_thread_chunk"] = oracle_chunk_one_thread(inp)
    if not args.no_other_configs and inp.name == DEFAULT_WORKLOAD:
        # the other workloads of the pages, measured briefly in the same run
        # (context beside the headline, not bench lines of their own)
        del H, ws, S, m
        torch.cuda.empty_cache()
        out["other_configs"] = {}
        flush = torch.empty(2 * INFINITY_CACHE_BYTES // 4, dtype=torch.float32, device=dev)
        for name in OTHER_CONFIGS:
            out["other_configs"][name] = measure_config(name, torch, dev, sa, flush=flush)
            torch.cuda.empty_cache()
        del flush
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
