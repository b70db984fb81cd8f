#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer on one MI355X.

Headline: prefill tokens/s of the Qwen3-Next-shaped layer (T = 4096, 16 key /
32 value heads, head dim 128, conv 4, gated RMSNorm, fp32 state), one step =
one gdn_prefill call over the whole batch, inputs resident in HBM, three
buffer sets rotated so that no step finds its inputs in the 256 MB cache.
The timed steps are plain calls.  Also reported: per-kernel times from a
separate pass of gdn_prefill_profiled calls (begin / end HIP events around
every kernel on its stream; those events cost about 40 us per call, which is
why they stay out of the timed steps), the roofline of the dominant kernel,
decode state GB/s (256 sequences, fp32 and bf16 state) and the fp64 CPU
oracle on a bounded sample as a baseline.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16 MFMA
FP32_PEAK = 157.3e12       # flop/s, fp32 (MFMA and vector ALUs alike)
D = 128
CHUNK = 64

# Algorithmic work per (token, value head), dense 64x64 tile count.
FLOP_SWEEP = 6 * D * D + 2 * CHUNK * D           # W S^T, Q S^T, K^T U, P U
FLOP_PREP = 2 * CHUNK * D + 2 * CHUNK * D + (2 * CHUNK * D + 2 * CHUNK * D) // 2  # W, U~, (KK^T, QK^T)/2
FLOP_LAYER = 180224                               # whole chunked layer
FLOP_LAYER_MIN = 139264                           # the same, triangular blocks skipped


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = ["gated_deltanet_layer_02_amd/csrc/gdn_prefill.hip",
                  "gated_deltanet_layer_02_amd/csrc/gdn_decode.hip",
                  "gated_deltanet_layer_02_amd/csrc/gdn_common.hpp",
                  "gated_deltanet_layer_02_amd/csrc/gdn_internal.hpp",
                  "gated_deltanet_layer_02_amd/build.py"]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    cur = source_hash(KERNEL_SOURCES)
    for line in open(path):
        m = re.match(r"\|\s*(\w+)\s*\|\s*([0-9a-f]{16})\s*\|\s*([0-9.eE+]+)\s*\|\s*([0-9.eE+]+)\s*\|", line)
        if m and m.group(1) == kernel and m.group(2) == cur:
            return float(m.group(3)) + float(m.group(4))
    return None


class Hip:
    """hipEvent API of the HIP runtime torch already loaded."""

    def __init__(self):
        self.l = ctypes.CDLL("libamdhip64.so.7")
        self.l.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.l.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.l.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.l.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.l.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.l.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.l.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, e):
        self.l.hipEventDestroy(e)


def clone_call(call):
    """Same inputs in fresh buffers (another buffer set for rotation)."""
    import copy
    c = copy.copy(call)
    for n in ("q", "k", "v", "g", "beta", "z", "conv_w", "norm_w", "initial_state",
              "conv_state_in", "out", "final_state", "conv_state_out", "workspace", "cu"):
        t = getattr(call, n)
        setattr(c, n, None if t is None else t.clone())
    return c


def bench_prefill(args, hip):
    import torch
    import gdn_synth as gs
    from gated_deltanet_layer_02_amd.binding import STAGE_NAMES
    from gated_deltanet_layer_02_amd.tensors import PrefillCall

    p = gs.configs()["C1"]
    log(f"[bench] generating {p.name} inputs")
    x = gs.generate(p)
    base = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True)
    sets = [base] + [clone_call(base) for _ in range(args.buffer_sets - 1)]
    stream = torch.cuda.current_stream().cuda_stream
    log(f"[bench] warmup {args.warmup} steps")
    for i in range(args.warmup):
        sets[i % len(sets)].run(stream=stream)
    torch.cuda.synchronize()

    # timed region: plain calls, HIP events on the launch stream at both ends
    log(f"[bench] timing {args.steps} steps")
    ev0, ev1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(ev0, stream)
    for i in range(args.steps):
        sets[i % len(sets)].run(stream=stream)
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_plain = hip.ms(ev0, ev1) / args.steps
    hip.destroy(ev0)
    hip.destroy(ev1)

    # per-kernel times: the same calls again with begin / end events around
    # every kernel (gdn_prefill_profiled); the events themselves cost time,
    # so these steps are not the timed ones
    nev = 2 + 2 * 8
    prof_steps = max(5, min(args.steps, 20))
    events = [[hip.event() for _ in range(nev)] for _ in range(prof_steps)]
    stage_ids = None
    log(f"[bench] {prof_steps} profiled steps for per-kernel times")
    for i in range(prof_steps):
        stage_ids = sets[i % len(sets)].run_profiled(events[i], stream=stream)
    torch.cuda.synchronize()

    # kernel i ran between ev[2 + 2i] and ev[3 + 2i] on its own stream; a
    # stage's time is the sum over its launches (launches of different
    # stages overlap when the call is split into chunk segments)
    stage_ms = {STAGE_NAMES[s]: 0.0 for s in stage_ids}
    launches = {STAGE_NAMES[s]: 0 for s in stage_ids}
    for s in stage_ids:
        launches[STAGE_NAMES[s]] += 1
    prof_ms = 0.0
    for ev in events:
        for j, s in enumerate(stage_ids):
            stage_ms[STAGE_NAMES[s]] += hip.ms(ev[2 + 2 * j], ev[3 + 2 * j]) / prof_steps
        prof_ms += hip.ms(ev[0], ev[1]) / prof_steps
    for ev in events:
        for e in ev:
            hip.destroy(e)
    gpu_ms = gpu_ms_plain

    T, Hv, Hk, N = p.T, p.Hv, p.Hk, p.N
    io_bytes = (2 * T * Hk * D + 3 * T * Hv * D) * 2 + 2 * T * Hv * 4 \
        + p.Cch * 4 * 2 + D * 2 + N * Hv * D * D * 4 + N * 3 * p.Cch * 2
    dominant = max(stage_ms, key=stage_ms.get)
    dom_s = stage_ms[dominant] * 1e-3
    # algorithmic flop per (token, value head) of the dominant kernel's share,
    # dense 64x64 tile count; the pipelined kernel runs the whole layer
    count = None
    if dominant == "state_sweep":
        count = ("sweep: W S^T, Q S^T, K^T U (6 d^2) + P U (2 C d)", FLOP_SWEEP)
    elif dominant == "chunk_prep":
        count = ("prep: T [b V | b gamma K] (4 C d) + half of K K^T and Q K^T", FLOP_PREP)
    elif dominant == "prep_sweep":
        count = ("whole layer: K K^T, Q K^T, T [b V | b gamma K], P U (10 C d) + 6 d^2", FLOP_LAYER)
    if count is not None:
        achieved, peak, unit, bound = count[1] * T * Hv / dom_s, MFMA_BF16_PEAK, "TFLOP/s", "mfma"
    else:   # gated norm: reads o and z, writes out
        achieved, peak, unit, bound = 3 * T * Hv * D * 2 / dom_s, HBM_PEAK, "GB/s", "hbm"
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    traffic = measured_traffic(dominant)
    nl = launches[dominant]
    roof = {"bound": bound, "achieved": round(achieved / scale, 2), "peak": peak / scale,
            "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": traffic,   # HBM bytes per launch (counter summary average)
            "flop_per_token_head": count[1] if count else None,
            "flop_count": count[0] if count else None,
            "flop_per_launch": count[1] * T * Hv if count else None,
            "kernel": dominant, "launches_per_step": nl,
            "kernel_us_per_launch": round(stage_ms[dominant] * 1e3 / nl, 2),
            "kernel_us_per_step": round(stage_ms[dominant] * 1e3, 2)}
    path = {"gpu_us_per_step": round(gpu_ms * 1e3, 2),
            "profiled_us_per_step": round(prof_ms * 1e3, 2),
            "hbm_algorithmic_bytes": io_bytes,
            "hbm_frac": round(io_bytes / (gpu_ms * 1e-3) / HBM_PEAK, 4),
            "mfma_frac_dense_tile": round(FLOP_LAYER * T * Hv / (gpu_ms * 1e-3) / MFMA_BF16_PEAK, 4)}
    return dict(p=p, x=x, ms_per_step=ms_per_step, tokens_per_s=T / (ms_per_step * 1e-3),
                stages_us={k: round(v * 1e3, 2) for k, v in stage_ms.items()},
                roofline=roof, path=path, buffer_sets=len(sets))


def bench_decode(args, hip, cfg):
    import torch
    import gdn_synth as gs
    from gated_deltanet_layer_02_amd.tensors import DecodeCall

    p = gs.configs()[cfg]
    log(f"[bench] decode {p.name}")
    x = gs.generate(p)
    dc = DecodeCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=p.state_dtype == gs.BF16)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        dc.run(stream=stream)
    torch.cuda.synchronize()
    reps = max(5, args.steps)
    # the decode loop: `reps` steps back to back between two events on the
    # stream (as the prefill line times its steps), then the same steps with
    # an event between every two calls for the per-call median
    ev0, ev1 = hip.event(), hip.event()
    hip.record(ev0, stream)
    for i in range(reps):
        dc.run(stream=stream)
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    t = hip.ms(ev0, ev1) * 1e-3 / reps
    hip.destroy(ev0)
    hip.destroy(ev1)
    evs = [hip.event() for _ in range(reps + 1)]
    hip.record(evs[0], stream)
    for i in range(reps):
        dc.run(stream=stream)
        hip.record(evs[i + 1], stream)
    torch.cuda.synchronize()
    times = sorted(hip.ms(evs[i], evs[i + 1]) for i in range(reps))
    for e in evs:
        hip.destroy(e)
    t_call = times[len(times) // 2] * 1e-3
    sb = 2 if p.state_dtype == gs.BF16 else 4
    state_bytes = 2 * p.N * p.Hv * D * D * sb
    other = (2 * p.N * p.Hk * D + 3 * p.N * p.Hv * D) * 2 + 2 * p.N * p.Hv * 4 \
        + 2 * p.N * 3 * p.Cch * 2 + p.Cch * 4 * 2
    traffic = measured_traffic("decode_" + p.state_dtype)
    return {"state_dtype": p.state_dtype, "us": round(t * 1e6, 2),
            "timing": f"{reps} decode steps back to back between two events on the stream",
            "us_per_call_median": round(t_call * 1e6, 2),
            "frac_per_call_median": round((state_bytes + other) / t_call / HBM_PEAK, 4),
            "state_GBps": round(state_bytes / t / 1e9, 1),
            "total_GBps": round((state_bytes + other) / t / 1e9, 1),
            "tokens_per_s": round(p.N / t, 1),
            "roofline": {"bound": "hbm", "achieved": round((state_bytes + other) / t / 1e9, 1),
                         "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": round((state_bytes + other) / t / HBM_PEAK, 4), "traffic": traffic}}


def time_calls(hip, calls, steps, warmup):
    """Average time of one call over `steps` rotating calls, HIP events on the stream."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        calls[i % len(calls)](stream)
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for i in range(steps):
        calls[i % len(calls)](stream)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    t = hip.ms(e0, e1) * 1e-3 / steps
    hip.destroy(e0)
    hip.destroy(e1)
    return t


def bench_options(args, hip, pres):
    """C1 prefill with bf16 state storage in a state pool and a snapshot every
    16 chunks (gdn_prefill_ex), multi-token decode (verify) of 4 draft tokens
    per sequence at the C4 shape, fp32 state, and one GPU's share of the C1
    layer under 2-, 4- and 8-way head parallelism."""
    import numpy as np
    import gdn_synth as gs
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, VerifyCall

    p, x = pres["p"], pres["x"]
    log("[bench] prefill with bf16 state pool and snapshots every 16 chunks")
    xb = dict(x, state=gs.f32_to_bf16_bits(np.zeros((2, p.Hv, 128, 128), np.float32)))
    calls = [PrefillCall(xb, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=True,
                         slots=np.array([1], np.int32), num_state_slots=2, snapshot_every=16,
                         snapshot_base=np.array([0], np.int32), num_snapshot_slots=3)
             for _ in range(args.buffer_sets)]
    t = time_calls(hip, [c.run for c in calls], args.steps, args.warmup)
    opts = {"workload": "C1 prefill, bf16 state in a 2-row pool, snapshots every 16 chunks",
            "us": round(t * 1e6, 2), "tokens_per_s": round(p.T / t, 1),
            "vs_plain": round((p.T / t) / pres["tokens_per_s"], 4)}
    del calls

    D = 4
    c4 = gs.configs()["C4"]
    pv = gs.Problem("verify", [D] * c4.N, init_state_std=0.01, conv_state_std=0.01, seed=c4.seed)
    log(f"[bench] verify: {c4.N} sequences x {D} draft tokens, fp32 state")
    xv = gs.generate(pv)
    vc = VerifyCall(xv, D=D, Hk=pv.Hk, Hv=pv.Hv, io_bf16=True, state_bf16=False)
    t = time_calls(hip, [vc.run], max(5, args.steps // 2), 3)
    state = pv.N * pv.Hv * 128 * 128 * 4                  # the batch's fp32 states
    # state read once, D checkpoints written, conv window read, D conv checkpoints
    # written, q, k, v, z, out of the D tokens
    moved = state * (1 + D) + pv.N * 3 * pv.Cch * 2 * (1 + D) \
        + (2 * pv.N * D * pv.Hk * 128 + 3 * pv.N * D * pv.Hv * 128) * 2
    ver = {"workload": f"verify, {pv.N} sequences x {D} draft tokens, 16 key / 32 value heads, fp32 state",
           "us": round(t * 1e6, 2), "tokens_per_s": round(pv.N * D / t, 1),
           "roofline": {"bound": "hbm", "achieved": round(moved / t / 1e9, 1), "peak": HBM_PEAK / 1e9,
                        "unit": "GB/s", "frac": round(moved / t / HBM_PEAK, 4),
                        "bytes": moved}}
    # one GPU's share of the C1 layer under 2-, 4- and 8-way head parallelism
    # (8 / 4 / 2 key heads, twice as many value heads, 4,096 tokens): the
    # default call (segment-parallel form) against the plain separate launches
    # (and of the 65,536-token layer with seeded states under 8-way parallelism)
    shares = {}
    for tp, Hk, T, name in ((2, 8, p.T, "tp2"), (4, 4, p.T, "tp4"), (8, 2, p.T, "tp8"),
                            (8, 2, 65536, "tp8_65536")):
        states = dict(init_state_std=0.01, conv_state_std=0.01) if T != p.T else {}
        ps = gs.Problem(f"{name}-share", [T], Hk=Hk, Hv=2 * Hk, seed=1001 + tp + T, **states)
        log(f"[bench] TP-{tp} share: {Hk} key / {2 * Hk} value heads, {T} tokens")
        xs = gs.generate(ps)
        row = {"workload": f"prefill, 1 sequence of {T} tokens, {Hk} key / {2 * Hk} value heads "
                           f"(one GPU's share of 16 / 32 under {tp}-way head parallelism)"
                           + (", seeded states" if states else "")}
        for label, sep in (("default", False), ("separate_launches", True)):
            calls = [PrefillCall(xs, Hk=Hk, Hv=2 * Hk, io_bf16=True, separate_launches=sep)
                     for _ in range(args.buffer_sets)]
            if label == "default":
                row["launch"] = launch_form(hip, calls[0])
            steps = args.steps if T == p.T else max(5, args.steps // 5)
            t = time_calls(hip, [c.run for c in calls], steps, min(args.warmup, steps))
            row[label] = {"us": round(t * 1e6, 2), "tokens_per_s": round(T / t, 1),
                          "flop_frac_dense_tile": round(FLOP_LAYER * T * 2 * Hk / t / MFMA_BF16_PEAK, 4)}
            del calls
        row["speedup"] = round(row["separate_launches"]["us"] / row["default"]["us"], 3)
        shares[name] = row
    # the serving stand-ins (93 new prompts of 250-350 tokens; a decode step of
    # 93 sequences, fp32 state)
    from gated_deltanet_layer_02_amd.binding import STAGE_NAMES
    from gated_deltanet_layer_02_amd.tensors import DecodeCall
    import torch
    sv = gs.serving()
    pp, pd = sv["prefill"], sv["decode"]
    log(f"[bench] serving: {pp.name}; {pd.name}")
    xp = gs.generate(pp)
    calls = [PrefillCall(xp, Hk=pp.Hk, Hv=pp.Hv, io_bf16=True) for _ in range(args.buffer_sets)]
    t = time_calls(hip, [c.run for c in calls], args.steps, args.warmup)
    stream = torch.cuda.current_stream().cuda_stream
    stages = {}
    for r in range(4):
        ev = [hip.event() for _ in range(2 + 2 * 16)]
        ids = calls[r % len(calls)].run_profiled(ev, stream=stream)
        torch.cuda.synchronize()
        if r > 0:
            for i, sid in enumerate(ids):
                stages.setdefault(STAGE_NAMES[sid], []).append(hip.ms(ev[2 + 2 * i], ev[3 + 2 * i]) * 1e3)
        for e in ev:
            hip.destroy(e)
    serve = {"prefill": {"workload": pp.name, "tokens": pp.T, "sequences": pp.N, "us": round(t * 1e6, 2),
                         "tokens_per_s": round(pp.T / t, 1), "launch": launch_form(hip, calls[0]),
                         "flop_frac_dense_tile": round(FLOP_LAYER * pp.T * pp.Hv / t / MFMA_BF16_PEAK, 4),
                         "hbm_frac": round(layer_bytes(pp) / t / HBM_PEAK, 4),
                         "stages_us_profiled": {k: round(sorted(v)[len(v) // 2], 2) for k, v in stages.items()}}}
    del calls
    xd = gs.generate(pd)
    dc = DecodeCall(xd, Hk=pd.Hk, Hv=pd.Hv, io_bf16=True, state_bf16=False)
    t = time_calls(hip, [dc.run], args.steps, args.warmup)
    d = pd.dk   # head dim (D above is the verify leg's draft count)
    moved = 2 * pd.N * pd.Hv * d * d * 4 + (2 * pd.N * pd.Hk * d + 3 * pd.N * pd.Hv * d) * 2 \
        + 2 * pd.N * pd.Hv * 4 + 2 * pd.N * 3 * pd.Cch * 2 + pd.Cch * 4 * 2
    serve["decode"] = {"workload": pd.name, "us": round(t * 1e6, 2), "tokens_per_s": round(pd.N / t, 1),
                       "total_GBps": round(moved / t / 1e9, 1), "hbm_frac": round(moved / t / HBM_PEAK, 4)}
    return {"prefill_pool_bf16_snapshots": opts, "verify": ver, "tp_shares": shares, "serving": serve}


def layer_bytes(p):
    """Once-each bytes of one prefill call: q, k, v, z, out, g, beta, weights,
    states and conv states in and out."""
    import gdn_synth as gs
    es = 2 if p.io == gs.BF16 else 4
    b = (2 * p.T * p.Hk * D + 2 * p.T * p.Hv * D) * es + 2 * p.T * p.Hv * 4
    if p.gate:
        b += p.T * p.Hv * D * es + D * es
    if p.conv:
        b += p.Cch * 4 * es + p.N * 3 * p.Cch * es * (2 if p.conv_state_std is not None else 1)
    b += p.N * p.Hv * D * D * 4 * (2 if p.init_state_std is not None else 1)
    return b


def time_each(hip, calls, steps, warmup):
    """Per-call times (s), HIP events around each call on the stream, calls rotated."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        calls[i % len(calls)](stream)
    torch.cuda.synchronize()
    ev = [(hip.event(), hip.event()) for _ in range(steps)]
    for i in range(steps):
        hip.record(ev[i][0], stream)
        calls[i % len(calls)](stream)
        hip.record(ev[i][1], stream)
    torch.cuda.synchronize()
    ts = sorted(hip.ms(a, b) * 1e-3 for a, b in ev)
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    return ts


def launch_form(hip, call):
    """Which form the library chose for this call (from a profiled call's stages)."""
    import torch
    from gated_deltanet_layer_02_amd.binding import STAGE_NAMES
    ev = [hip.event() for _ in range(2 + 2 * 8)]
    ids = call.run_profiled(ev, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for e in ev:
        hip.destroy(e)
    names = [STAGE_NAMES[i] for i in ids]
    if "prep_sweep" in names:
        return "pipelined"
    return "segments" if "seg_compose" in names else "separate launches"


def bench_configs(args, hip):
    """Every prefill configuration: per-call median / p10 / p90, tokens/s, MFMA
    fractions (dense-tile and triangle-aware counts) and HBM fraction; the time
    per token of C2 against C1 (the layer is O(T)); and reference peaks
    measured on this GPU (a device copy, and torch's bf16 GEMM)."""
    import torch
    import gdn_synth as gs
    from gated_deltanet_layer_02_amd.tensors import PrefillCall

    out = {}
    per_token = {}
    for name in ("C0", "C1", "C2", "C3"):
        p = gs.configs()[name]
        log(f"[bench] config {name}: {p.N} sequence(s), {p.T} tokens, io {p.io}")
        x = gs.generate(p)
        sets = 3 if p.T <= 8192 else 1
        calls = [PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=p.io == gs.BF16, l2norm=p.l2norm, scale=p.scale,
                             l2_eps=p.l2_eps, norm_eps=p.norm_eps) for _ in range(sets)]
        form = launch_form(hip, calls[0])
        steps = 30 if p.T <= 8192 else 10
        ts = time_each(hip, [c.run for c in calls], steps, 5)
        med, p10, p90 = ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]
        byt = layer_bytes(p)
        fpeak = MFMA_BF16_PEAK if p.io == gs.BF16 else FP32_PEAK   # fp32 I/O computes in fp32
        per_token[name] = med / p.T
        out[name] = {"tokens": p.T, "sequences": p.N, "io": p.io, "launch": form,
                     "us_median": round(med * 1e6, 2), "us_p10": round(p10 * 1e6, 2),
                     "us_p90": round(p90 * 1e6, 2), "tokens_per_s": round(p.T / med, 1),
                     "flop_peak_TFLOPs": fpeak / 1e12,
                     "flop_frac_dense_tile": round(FLOP_LAYER * p.T * p.Hv / med / fpeak, 4),
                     "flop_frac_triangle_aware": round(FLOP_LAYER_MIN * p.T * p.Hv / med / fpeak, 4),
                     "hbm_frac": round(byt / med / HBM_PEAK, 4), "bytes": byt}
        del calls, x
        torch.cuda.empty_cache()
    out["time_per_token_C2_over_C1"] = round(per_token["C2"] / per_token["C1"], 3)

    # reference peaks on this GPU (torch plumbing: a device copy and a bf16 GEMM)
    stream = torch.cuda.current_stream().cuda_stream
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ts = time_each(hip, [lambda s: dst.copy_(src)], 10, 3)
    copy = 2 * src.numel() / ts[len(ts) // 2]
    del src, dst
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    ts = time_each(hip, [lambda s: torch.matmul(a, b)], 10, 3)
    gemm = 2 * 8192 ** 3 / ts[len(ts) // 2]
    del a, b
    torch.cuda.empty_cache()
    out["measured_peaks"] = {"device_copy_GBps": round(copy / 1e9, 1),
                             "torch_bf16_gemm_8192_TFLOPs": round(gemm / 1e12, 1)}
    return out


def _host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _prefix(x, S):
    """The first S tokens of a single-sequence problem's inputs."""
    import numpy as np
    xs = {n: (a[:S] if n in ("q", "k", "v", "z", "g", "beta") else a) for n, a in x.items()}
    xs["cu_seqlens"] = np.array([0, S], dtype=np.int32)
    return xs


def cpu_baseline_configs(per_run_s: float = 1.0):
    """The fp64 oracle on every configuration, with one host thread and with
    all of them: tokens/s on a bounded sample of each (about per_run_s of
    single-thread work), the sample stated."""
    import dataclasses
    import numpy as np
    import gdn_synth as gs
    from oracle import oracle
    allthreads = oracle.max_threads()
    res = {"host_cpu": _host_cpu(), "host_logical_cpus": os.cpu_count(), "threads_all": allthreads}
    for name in ("C0", "C1", "C2", "C3", "C4", "C4b"):
        p = gs.configs()[name]
        x = gs.generate(p)
        if p.decode:
            sample, xs, ps, tokens = f"all {p.N} sequences, one token each", x, p, p.N
        elif p.N == 1 and p.T <= 512:
            sample, xs, ps, tokens = f"all {p.T} tokens", x, p, p.T
        else:
            # the first S tokens of the first sequence, S sized for about
            # per_run_s of single-thread work on all value heads
            L0 = p.seq_lens[0]
            x0 = {n: a for n, a in x.items()}
            if p.N > 1:
                t1 = int(x["cu_seqlens"][1])
                x0 = {n: (a[:t1] if n in ("q", "k", "v", "z", "g", "beta") else a) for n, a in x.items()}
                x0["state"] = None if x["state"] is None else x["state"][:1]
                x0["conv_state"] = None if x["conv_state"] is None else x["conv_state"][:1]
            S = min(L0, 64)
            t = _time_oracle(oracle, dataclasses.replace(p, seq_lens=[S]), _prefix(x0, S), 1)
            S = int(min(L0, max(64, S * per_run_s / max(t, 1e-3))))
            ps, xs, tokens = dataclasses.replace(p, seq_lens=[S]), _prefix(x0, S), S
            sample = f"first {S} tokens of sequence 0 ({L0} tokens), all {p.Hv} value heads"
        entry = {"sample": sample}
        for label, th in (("one_thread", 1), ("all_threads", allthreads)):
            reps, t = 0, 0.0
            while reps < 20 and (t < per_run_s or reps < 2):
                t += _time_oracle(oracle, ps, xs, th)
                reps += 1
            used = min(th, ps.N * ps.Hv)
            entry[label] = {"tokens_per_s": round(reps * tokens / t, 2), "threads": used,
                            "runs": reps, "seconds": round(t, 2)}
        res[name] = entry
        log(f"[bench] cpu oracle {name}: {entry['one_thread']['tokens_per_s']} tok/s (1 thread), "
            f"{entry['all_threads']['tokens_per_s']} tok/s ({entry['all_threads']['threads']} threads)")
    return res


def _time_oracle(oracle, p, xs, threads):
    t0 = time.perf_counter()
    oracle.run_problem(p, xs, threads=threads)
    return time.perf_counter() - t0


def cpu_baseline(pres, target_s: float):
    """The fp64 oracle on the first S tokens of the same C1 inputs, all heads."""
    import numpy as np
    from oracle import oracle
    p, x = pres["p"], pres["x"]

    def run(S):
        xs = _prefix(x, S)
        t0 = time.perf_counter()
        oracle.run_problem(p, xs)
        return time.perf_counter() - t0

    S = 64
    t = run(S)
    S = int(min(p.T, max(64, S * target_s / max(t, 1e-3))))
    log(f"[bench] cpu baseline: oracle on {S} tokens x {p.Hv} heads")
    # repeat the sample until about target_s of wall time (at most 50 times)
    reps, t = 0, 0.0
    while reps < 50 and (t < target_s or reps < 3):
        t += run(S)
        reps += 1
    threads = min(oracle.max_threads(), p.N * p.Hv)
    cpu = _host_cpu()
    return {"value": round(reps * S / t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {p.T} tokens of the same workload, all {p.Hv} value heads, "
                      f"fp64, OpenMP over heads, {reps} runs in {t:.1f} s wall",
            "host_cpu": cpu, "host_logical_cpus": os.cpu_count()}


def calibrate_mfma(blocks: int = 1024, iters: int = 256):
    """The MFMA loops of libgdn_calib.so (counter calibration): blocks x 4 waves
    x iters x 8 MFMA instructions of each kind, 16x16x32 bf16 (16,384 flop)
    then 16x16x16 bf16 (8,192 flop)."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_deltanet_layer_02_amd", "libgdn_calib.so"))
    lib.gdn_calib_mfma.restype = ctypes.c_int
    lib.gdn_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for kind in (0, 1):
        assert lib.gdn_calib_mfma(kind, blocks, iters, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        n = blocks * 4 * iters * 8
        log(f"[bench] calibration MFMA loop kind {kind}: {n} instructions, "
            f"{n * (16384 if kind == 0 else 8192)} flop")


def run_only(args, hip, name):
    """One configuration's prefill alone (for counter runs): warmup + steps
    calls on one buffer set, the median printed as a JSON line."""
    import gdn_synth as gs
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    p = gs.configs()[name]
    log(f"[bench] only {name}: {p.N} sequence(s), {p.T} tokens")
    x = gs.generate(p)
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=p.io == gs.BF16, l2norm=p.l2norm, scale=p.scale,
                       l2_eps=p.l2_eps, norm_eps=p.norm_eps)
    ts = time_each(hip, [call.run], args.steps, args.warmup)
    print(json.dumps({"config": name, "tokens": p.T, "launch": launch_form(hip, call),
                      "calls": args.steps, "us_median": round(ts[len(ts) // 2] * 1e6, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--buffer-sets", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=5.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the prefill-options and verify legs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration prefill timings (C0-C3) and reference peaks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 512 MiB device-to-device copy first (counter calibration)")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="run the MFMA loops of libgdn_calib.so first (counter calibration)")
    ap.add_argument("--only", choices=["C0", "C1", "C2", "C3"],
                    help="time one prefill configuration alone (counter runs) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    hip = Hip()

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 512 MiB device-to-device")
        del src, dst
    if args.calibrate_mfma:
        calibrate_mfma()
    if args.only:
        run_only(args, hip, args.only)
        return

    pres = bench_prefill(args, hip)
    dec = None
    if not args.no_decode:
        dec = {"metric": "decode state GB/s", "fp32_state": bench_decode(args, hip, "C4"),
               "bf16_state": bench_decode(args, hip, "C4b")}
    opts = None if args.no_options else bench_options(args, hip, pres)
    cfgs = None if args.no_configs else bench_configs(args, hip)
    cpu = None if args.no_cpu_baseline else cpu_baseline(pres, args.cpu_seconds)
    cpu_cfg = None if args.no_cpu_baseline else cpu_baseline_configs()

    p = pres["p"]
    line = {
        "metric": "GatedDeltaNet prefill tokens/s (T=4096, 16k/32v heads)",
        "value": round(pres["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pres["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill, 1 sequence of 4096 tokens, 16 key / 32 value heads, "
                               "head dim 128, conv 4 + SiLU, L2 q/k, z-gated RMSNorm, fp32 state",
                   "T": p.T, "num_seqs": p.N, "Hk": p.Hk, "Hv": p.Hv, "chunk": CHUNK,
                   "io": "bf16", "state": "fp32", "buffer_sets": pres["buffer_sets"]},
        "roofline": pres["roofline"],
        "cpu_baseline": cpu,
        "cpu_baseline_configs": cpu_cfg,
        "stages_us": pres["stages_us"],
        "path": pres["path"],
        "decode": dec,
        "options": opts,
        "configs": cfgs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
