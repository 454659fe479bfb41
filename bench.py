"""Benchmark of the ReplaySSM decode path on one MI355X.

Default workload (the headline): one Mamba-2-shaped SSM layer in standard
decode -- batch 256, 128 heads, 8 groups, P=64, N=128, ring L=16, bf16
q/k/v, float32 checkpoint.  One step = append one token per sequence, the
output-only decode of that token, and the flush of every ring that became
full (every 16th step).  The timed region is K steps (default 256 = 16
windows) with all inputs resident in HBM; the eager per-token baseline is
timed the same way on the same inputs.

Prints ONE JSON line.  `roofline` is the fused step kernel (the dominant
one): algorithmic bytes per launch / its average duration, from HIP events
on the launch stream around whole windows of launches run after the timed
region (so the figure does not depend on --steps).  `cpu_baseline` is the float64 oracle on a bounded sample of
the same workload, timed on the host cores.

Other workloads (--workload verify | dual | stacked) print their own line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "SSM-layer decode tokens/s at B=256 + achieved HBM GB/s (% peak) vs eager"
HBM_PEAK_GBS = 8000.0
POOL_STEPS = 32   # distinct pre-generated input steps, cycled (values do not change the work)


# ---------------------------------------------------------------------------
# algorithmic byte model (bytes the method must move; cache re-reads and
# group-shared k/q counted once per group)
def state_bytes(w, st_bytes=4):
    return int(w.batch * w.heads * w.head_dim * w.state_dim * st_bytes)


def scale_bytes(w, st_bytes):
    """Scales of a copy: e4m3 one float per head, MX FP4 one byte per 32 values."""
    if st_bytes == 1:
        return w.batch * w.heads * 4
    if st_bytes == 0.5:
        return w.batch * w.heads * w.head_dim * w.state_dim // 32
    return 0


def decode_bytes(w, count, W=1, st_bytes=4, io=2):
    """One decode/verify launch with `count` live entries per sequence."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io          # v, (dt, a), k
    return (state_bytes(w, st_bytes) + scale_bytes(w, st_bytes)
            + B * (count * per_entry + W * G * N * io + W * H * P * 4))   # + q + y


def flush_bytes(w, count, copy_bytes=0, io=2):
    """Fold of `count` entries: the master read and written, the copy (and its
    scales) written; copy_bytes = bytes per value of the copy (0: none)."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io
    s = state_bytes(w)
    return 2 * s + B * count * per_entry + (state_bytes(w, copy_bytes) + scale_bytes(w, copy_bytes)
                                            if copy_bytes else 0)


def step_bytes(w, count, fold, io=2):
    """One fused step launch; `count` includes this step's token, which is read
    from the inputs and written to the ring."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io
    token = H * P * io + H * 8 + 2 * G * N * io          # v, (dt, a), q, k of the new token
    return (state_bytes(w) * (2 if fold else 1)
            + B * ((count - 1) * per_entry + 2 * token + H * P * 4))


def step_copy_bytes(w, count, st_bytes, io=2):
    """One copy-mode step launch (append + output-only decode from a copy of
    st_bytes bytes per value); `count` includes this step's token."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io
    token = H * P * io + H * 8 + 2 * G * N * io
    return (state_bytes(w, st_bytes) + scale_bytes(w, st_bytes)
            + B * ((count - 1) * per_entry + 2 * token + H * P * 4))


def verify_step_bytes(w, before, W, io=2):
    """One fused verify-round launch; `before` = ring counts per sequence at
    the start of the round (a sequence with count >= L-W+1 folds first: its
    checkpoint is written and its entries read by the fold; otherwise they
    are read by the ring term).  The drafts are read from the inputs and
    written to the ring."""
    B, H, G, P, N, L = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len
    per_entry = H * P * io + H * 8 + G * N * io
    token = H * P * io + H * 8 + 2 * G * N * io
    folds = int(np.sum(before >= L - W + 1))
    return (state_bytes(w) * (1 + folds / B)
            + float(np.sum(before)) * per_entry + B * (2 * W * token + W * H * P * 4))


def flop_model(P, N):
    """Multiply-adds one ring entry costs to reach the outputs (page
    "ReplaySSM: Cachear Inputs, No Estado", "Los dos caminos"): the state
    route builds the outer product v k^T into the state (P*N), the
    output-only route takes k . q (N) and adds the scaled v (P).  Their ratio
    P*N / (P + N) is 64 at P = N = 128, the pages' figure."""
    return {"state_route_macs_per_entry": P * N, "output_only_macs_per_entry": P + N,
            "ratio": P * N / (P + N), "ratio_at_128x128": 128 * 128 / 256}


def verify_step_copy_bytes(w, before, W, st_bytes, io=2):
    """One fused verify-round launch with a low-precision read copy: a
    sequence without a fold reads the copy (and its scales); one that folds
    reads and writes the float32 master and writes the copy (and scales).
    Ring entries, drafts and outputs as for verify_step_bytes."""
    B, H, G, P, N, L = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len
    per_entry = H * P * io + H * 8 + G * N * io
    token = H * P * io + H * 8 + 2 * G * N * io
    folds = int(np.sum(before >= L - W + 1))
    copy_seq = (state_bytes(w, st_bytes) + scale_bytes(w, st_bytes)) / B
    fold_seq = 2 * state_bytes(w) / B + copy_seq
    return (folds * fold_seq + (B - folds) * copy_seq
            + float(np.sum(before)) * per_entry + B * (2 * W * token + W * H * P * 4))


def eager_bytes(w, io=2):
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    return 2 * state_bytes(w) + B * (H * P * io + H * 8 + 2 * G * N * io + H * P * 4)


# ---------------------------------------------------------------------------
def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def input_pool(w, nsteps, t0=0):
    """nsteps seeded steps, resident on the device: q,k [T][B][G][N] ...
    (the seeded recipe evaluated on the device)."""
    return synth.step_inputs_torch(w, t0, t0 + nsteps, device="cuda")


def cpu_baseline(w, target_s=15.0, steps=256, chunk=32, rule="ssd", distinct=64):
    """The oracle, as it stands, on a bounded sample of the workload: the
    first `nseq` sequences, nseq chosen from a short calibration so the
    sample takes about target_s seconds of host time.  When the whole batch
    fits in that, the sample runs more than `steps` steps, cycling the inputs
    of the first `distinct` steps (as the device run cycles its own).
    Inputs are generated outside the timed calls."""
    import oracle
    from oracle import runs
    gen = synth.gdn_inputs if rule == "gdn" else synth.step_inputs

    def inputs(nseq, T):
        return [runs.widen_inputs(gen(w, t0, min(T, t0 + chunk), seqs=list(range(nseq))), w.io_dtype)
                for t0 in range(0, T, chunk)]

    def run(xs, T, S):
        total = 0.0
        for c in range((T + chunk - 1) // chunk):
            c0 = time.perf_counter()
            runs.standard(xs[c % len(xs)], S, rule=rule)
            total += time.perf_counter() - c0
        return total

    cal_seq, cal_T = 4, 32
    cal = run(inputs(cal_seq, cal_T), cal_T, np.zeros((cal_seq, w.heads, w.head_dim, w.state_dim)))
    per_token = cal / (cal_seq * cal_T)
    nseq = int(max(4, min(w.batch, target_s / (per_token * steps))))
    T = steps
    if nseq == w.batch:
        T = int(min(8 * steps, max(steps, target_s / (per_token * nseq))) // chunk * chunk)
    xs = inputs(nseq, min(T, distinct))
    S = np.zeros((nseq, w.heads, w.head_dim, w.state_dim))
    dt = run(xs, T, S)
    del xs, S
    cores = oracle.threads()
    # the same oracle on one core, over a smaller sample (first 16 sequences x 64 steps)
    n1, t1 = min(16, w.batch), min(64, steps)
    xs1 = inputs(n1, t1)
    oracle.set_threads(1)
    try:
        dt1 = run(xs1, t1, np.zeros((n1, w.heads, w.head_dim, w.state_dim)))
    finally:
        oracle.set_threads(cores)
    cyc = f" (the first {min(T, distinct)} steps' inputs cycled)" if T > distinct else ""
    return {"value": nseq * T / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 eager recurrence ({'gated delta rule' if rule == 'gdn' else 'Mamba-2'}), "
                      f"first {nseq} of {w.batch} sequences x {T} steps{cyc} "
                      f"of the same layer ({dt:.1f} s host time, input generation excluded)",
            "one_core": {"value": n1 * t1 / dt1, "unit": "tokens/s", "cores": 1,
                         "sample": f"first {n1} sequences x {t1} steps ({dt1:.1f} s host time)"}}


def _counter_traffic(kernel_files, summary_name):
    """HBM bytes per launch measured by rocprofv3 counters, if the summary in
    profiles/ was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", summary_name)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in kernel_files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


DECODE_SOURCES = ["linear_attention_decode_amd/csrc/decode_impl.h",
                  "linear_attention_decode_amd/csrc/ring_mx.h",
                  "linear_attention_decode_amd/csrc/device_common.h",
    "linear_attention_decode_amd/csrc/internal.h"]
STEP_SOURCES = ["linear_attention_decode_amd/csrc/step.hip",
                "linear_attention_decode_amd/csrc/step_common.h",
                "linear_attention_decode_amd/csrc/ring_mx.h",
                "linear_attention_decode_amd/csrc/device_common.h",
    "linear_attention_decode_amd/csrc/internal.h"]
STEP_COPY_SOURCES = ["linear_attention_decode_amd/csrc/step_copy.hip",
                     "linear_attention_decode_amd/csrc/step_common.h",
                     "linear_attention_decode_amd/csrc/decode_impl.h",
                     "linear_attention_decode_amd/csrc/ring_mx.h",
                     "linear_attention_decode_amd/csrc/device_common.h",
    "linear_attention_decode_amd/csrc/internal.h"]
GDN_SOURCES = ["linear_attention_decode_amd/csrc/gdn.hip",
               "linear_attention_decode_amd/csrc/decode_impl.h",
               "linear_attention_decode_amd/csrc/ring_mx.h",
               "linear_attention_decode_amd/csrc/device_common.h",
    "linear_attention_decode_amd/csrc/internal.h"]
VERIFY_STEP_SOURCES = ["linear_attention_decode_amd/csrc/verify_step.hip",
                       "linear_attention_decode_amd/csrc/wide_mx.h",
                       "linear_attention_decode_amd/csrc/step_common.h",
                       "linear_attention_decode_amd/csrc/ring_mx.h",
                       "linear_attention_decode_amd/csrc/device_common.h",
    "linear_attention_decode_amd/csrc/internal.h"]
VERIFY_WIDE_SOURCES = ["linear_attention_decode_amd/csrc/verify_wide.hip",
                       "linear_attention_decode_amd/csrc/wide_mx.h",
                       "linear_attention_decode_amd/csrc/decode_impl.h",
                       "linear_attention_decode_amd/csrc/ring_mx.h",
                       "linear_attention_decode_amd/csrc/device_common.h",
    "linear_attention_decode_amd/csrc/internal.h"]


def read_ceiling_gbs(nbytes=1 << 30, reps=96):
    """Read-bandwidth ceiling measured by the library's stream probe (mode 0:
    32 KiB tiles, all loads in flight, non-temporal), median of reps passes
    (96 x 1 GiB: about 15 ms of sustained reads)."""
    import torch
    import linear_attention_decode_amd as lad
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty((nbytes + 32767) // 32768, dtype=torch.float32, device="cuda")
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        lad.replay_stream_probe(0, src, dst, nbytes)
        e.record()
        ts.append((s, e))
    torch.cuda.synchronize()
    us = sorted(s.elapsed_time(e) * 1e3 for s, e in ts)[reps // 2]
    del src, dst
    torch.cuda.empty_cache()
    return nbytes / us / 1e3


def _bench_eager(args, w, pool, y):
    """The eager per-token baseline on the same inputs, timed like the steps."""
    import torch
    import linear_attention_decode_amd as lad
    B, H, G, P, N, L = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len
    cfg = lad.ReplayConfig(B, H, G, P, N, L, lad.BF16, lad.NONE, 0)
    S = torch.zeros((B, H, P, N), dtype=torch.float32, device="cuda")

    def estep(t):
        i = t % POOL_STEPS
        lad.replay_eager_step(cfg, S, S, pool["q"][i], pool["k"][i], pool["v"][i], pool["dt"][i],
                              pool["a"][i], y)
    for t in range(args.warmup):
        estep(t)
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for k in range(args.steps):
        estep(args.warmup + k)
    torch.cuda.synchronize()
    e1 = time.perf_counter()
    eager_tps = B * args.steps / (e1 - e0)
    eager_gbs = eager_bytes(w) * args.steps / (e1 - e0) / 1e9
    del S
    torch.cuda.empty_cache()
    return {"value": eager_tps, "unit": "tokens/s", "ms_per_step": 1e3 * (e1 - e0) / args.steps,
            "achieved_GBs": eager_gbs}



# ---------------------------------------------------------------------------
def bench_decode(args):
    import torch
    import linear_attention_decode_amd as lad

    w = synth.named("decode")
    B, H, G, P, N, L = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len
    rc = {"f32": None, "bf16": "bf16", "fp8": "fp8", "fp4": "fp4"}[args.read]
    st_bytes = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5}[args.read]
    copy_step = args.api == "step" and rc is not None   # the copy-mode step (+ the flush kernel on folds)
    pool = input_pool(w, POOL_STEPS)
    layer = lad.ReplayLayer(B, H, G, P, N, L, io_dtype="bf16", read_copy=rc)
    y = torch.empty((B, H, P), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(t, ev=None):
        i = t % POOL_STEPS
        args_t = (pool["q"][i], pool["k"][i], pool["v"][i], pool["dt"][i], pool["a"][i])
        if args.api == "step":
            # one fused launch: append + decode, or append + fold when the ring fills
            if ev is not None:
                ev[0].record(stream)
            layer.step(*args_t, y, flush_at=L)
            if ev is not None:
                ev[1].record(stream)
            return
        layer.append(1, *args_t)
        if ev is not None:
            ev[0].record(stream)
        layer.decode(y)
        if ev is not None:
            ev[1].record(stream)
        if (t + 1) % L == 0 and ev is not None:
            ev[2].record(stream)
            layer.flush(L)
            ev[3].record(stream)
        else:
            layer.flush(L)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    # The timed region: K steps with nothing recorded between launches, and
    # one pair of HIP events on the launch stream around the whole region.
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for k in range(args.steps):
        step(args.warmup + k)
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    region_s = r0.elapsed_time(r1) / 1e3
    timed_counts = [((args.warmup + k) % L) + 1 for k in range(args.steps)]
    folds_timed = sum(1 for c in timed_counts if c >= L)

    # The roofline pass, after the timed region and independent of K: the
    # steps continue to the next window start, then `reps` whole windows
    # (ring counts 1..L each, the fold included, as in the schedule) run back
    # to back between one pair of events -> the kernel's average launch time
    # over the schedule.  Then one more window with every launch between its
    # own events gives the two routes apart (an event between two launches
    # holds the second back by a few microseconds, so these read a little slow).
    t = args.warmup + args.steps
    while t % L != 0:
        step(t)
        t += 1
    reps = max(1, args.roofline_windows)
    if args.api == "step":
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for i in range(reps * L):
            step(t + i)
        p1.record(stream)
        t += reps * L
    route_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(L)]
    for i in range(L):
        step(t + i, route_evs[i])
    torch.cuda.synchronize()
    word, _ = layer.get_error()
    assert word == 0, f"device error bits {word}"
    counts = list(range(1, L + 1))
    if copy_step:
        # launches of the copy-mode step; the fold step's bracket holds the flush kernel too
        def launch_bytes(c, fold):
            return step_copy_bytes(w, c, st_bytes) + (flush_bytes(w, c, st_bytes) if fold else 0)
    else:
        def launch_bytes(c, fold):
            return step_bytes(w, c, fold)
    if args.api == "step":
        # the dominant kernel is the fused step kernel itself
        pass_s = p0.elapsed_time(p1) / 1e3
        kernel_bytes = reps * sum(launch_bytes(c, c >= L) for c in counts)
        kernel_time = pass_s
        n_launch = reps * L
        avg_us = 1e6 * pass_s / n_launch
        step_ms = [e[0].elapsed_time(e[1]) for e in route_evs]
        folds = [c >= L for c in counts]
        dec_ms = [m for m, f in zip(step_ms, folds) if not f]
        fl_ms = [m for m, f in zip(step_ms, folds) if f]
        kernel_name = ("copy-mode step (append + output-only decode from the copy; the flush kernel after it "
                       "on full rings)" if copy_step else
                       "step (append + output-only decode, or append + fold on full rings)")
        by_route = {}
        for route, sel in (("output_only", False), ("fold", True)):
            b_r = sum(launch_bytes(c, f) for c, f in zip(counts, folds) if f == sel)
            t_r = sum(m for m, f in zip(step_ms, folds) if f == sel) / 1e3
            by_route[route] = {"achieved": b_r / t_r / 1e9, "frac": b_r / t_r / 1e9 / HBM_PEAK_GBS,
                               "launches": sum(1 for f in folds if f == sel),
                               "avg_launch_us": 1e6 * t_r / sum(1 for f in folds if f == sel)}
        region_bytes = sum(launch_bytes(c, c >= L) for c in timed_counts)
    else:
        dec_ms = [e[0].elapsed_time(e[1]) for e in route_evs]
        fl_ms = [route_evs[L - 1][2].elapsed_time(route_evs[L - 1][3])]
        kernel_bytes = sum(decode_bytes(w, c, 1, st_bytes) for c in counts)
        kernel_time = sum(dec_ms) / 1e3
        n_launch = L
        avg_us = 1e3 * sum(dec_ms) / len(dec_ms)
        kernel_name = "decode (output-only)"
        by_route = None
        region_bytes = None
    achieved = kernel_bytes / kernel_time / 1e9
    layer.close()
    del layer
    torch.cuda.empty_cache()

    eager_out = None if args.no_eager else _bench_eager(args, w, pool, y)
    ceiling = args.read_ceiling

    window_replay = sum(decode_bytes(w, c, 1, st_bytes) for c in range(1, L + 1)) \
        + flush_bytes(w, L, 0 if st_bytes == 4 else st_bytes) \
        + B * L * 2 * (H * P * 2 + H * 8 + 2 * G * N * 2)            # appends: read input + write ring
    window_eager = L * eager_bytes(w)
    if copy_step:
        traffic = _counter_traffic(STEP_COPY_SOURCES, f"step_copy_fused_kernel_{args.read}_b256_h128_counters.txt")
    elif args.api == "step":
        traffic = _counter_traffic(STEP_SOURCES, "step_kernel_f32_b256_h128_counters.txt")
    else:
        traffic = _counter_traffic(DECODE_SOURCES, f"decode_kernel_{args.read}_b256_h128_counters.txt")
    out = {
        "metric": METRIC,
        "value": B * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": f"synthetic (seeded SplitMix64/Box-Muller, {POOL_STEPS} distinct steps cycled)",
        "config": {"workload": "Mamba-2-shaped SSM layer, standard decode", "batch": B, "heads": H,
                   "groups": G, "head_dim": P, "state_dim": N, "ring_len": L, "io": "bf16",
                   "checkpoint": "f32", "read_copy": args.read, "flush_every": L, "api": args.api},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel_name, "avg_launch_us": avg_us, "timed_launches": n_launch,
                     "launches_from": (f"{reps} whole windows (ring counts 1..{L}, one fold each) back to back "
                                       "after the timed region, one pair of HIP events around them"
                                       if args.api == "step" else
                                       f"one window (ring counts 1..{L}), each decode launch between HIP events"),
                     "algorithmic_bytes_per_launch": kernel_bytes / n_launch,
                     "read_ceiling_GBs": ceiling, "frac_of_read_ceiling": achieved / ceiling,
                     "by_route": by_route},
        "timed_region": {"folds": folds_timed, "fold_fraction": folds_timed / args.steps,
                         "schedule_fold_fraction": 1.0 / L,
                         "event_ms": 1e3 * region_s,
                         "achieved_GBs": (region_bytes / region_s / 1e9) if region_bytes else None},
        "flop_model": flop_model(P, N),
        ("output_only_launch_avg_us" if args.api == "step" else "decode_avg_us"):
            1e3 * sum(dec_ms) / max(1, len(dec_ms)),
        ("fold_launch_avg_us" if args.api == "step" else "flush_avg_us"):
            1e3 * sum(fl_ms) / max(1, len(fl_ms)),
        "eager": eager_out,
        "speedup_vs_eager": (B * args.steps / elapsed) / eager_out["value"] if eager_out else None,
        "window_bytes_ratio_vs_eager": window_replay / window_eager,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    return out



# ---------------------------------------------------------------------------
def bench_gdn(args):
    """Gated DeltaNet layer (B=256, H=32 value heads over G=16 key heads,
    P=N=128, L=16, bf16 q/k/v, float32 checkpoint; unit-length q, k, sigmoid
    beta): standard decode through replay_step (append, the output-only
    route -- the backward chain over the ring and one pass over S0 -- and
    the fold when the ring is full), against the layer's eager step
    (S_t written every token) on the same inputs.  With --read bf16/fp8/fp4
    the outputs read a copy of that precision (separated: the fold writes the
    float32 checkpoint and the copy).  The roofline pass runs one more window
    as separate calls with HIP events around each output-only launch and the
    fold."""
    import torch
    import linear_attention_decode_amd as lad

    w = synth.named("gdn")
    B, H, G, P, N, L = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len
    pool = synth.gdn_inputs_torch(w, 0, POOL_STEPS, device="cuda")
    read = None if args.read == "f32" else args.read
    st_bytes = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5}[args.read]
    layer = lad.ReplayLayer(B, H, G, P, N, L, io_dtype="bf16", rule="gdn", read_copy=read)
    y = torch.empty((B, H, P), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def args_t(t):
        i = t % POOL_STEPS
        return (pool["q"][i], pool["k"][i], pool["v"][i], pool["dt"][i], pool["a"][i])

    for t in range(args.warmup):
        layer.step(*args_t(t), y, flush_at=L)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        layer.step(*args_t(args.warmup + k), y, flush_at=L)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # roofline pass: to the next window start, then `reps` windows as calls
    t = args.warmup + args.steps
    while t % L != 0:
        layer.step(*args_t(t), y, flush_at=L)
        t += 1
    reps = max(1, args.roofline_windows)
    dec_ev, fold_ev = _events(reps * L), _events(reps)
    for i in range(reps * L):
        layer.append(1, *args_t(t + i))
        dec_ev[i][0].record(stream)
        layer.decode(y)
        dec_ev[i][1].record(stream)
        if (i + 1) % L == 0:
            fold_ev[i // L][0].record(stream)
            layer.flush(L)
            fold_ev[i // L][1].record(stream)
    torch.cuda.synchronize()
    word, _ = layer.get_error()
    assert word == 0, f"device error bits {word}"
    dec_s = sum(e[0].elapsed_time(e[1]) for e in dec_ev) / 1e3
    fold_s = sum(e[0].elapsed_time(e[1]) for e in fold_ev) / 1e3
    dec_bytes = reps * sum(decode_bytes(w, c, st_bytes=st_bytes) for c in range(1, L + 1))
    fold_bytes = reps * flush_bytes(w, L, copy_bytes=0 if read is None else st_bytes)
    achieved = dec_bytes / dec_s / 1e9
    layer.close()
    del layer
    torch.cuda.empty_cache()

    # the layer's eager step on the same inputs
    cfg = lad.ReplayConfig(B, H, G, P, N, L, lad.BF16, lad.NONE, 0, lad.GATED_DELTA)
    S = torch.zeros((B, H, P, N), dtype=torch.float32, device="cuda")
    eager_out = None
    if not args.no_eager:
        for t in range(args.warmup):
            lad.replay_eager_step(cfg, S, S, *args_t(t), y)
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        for k in range(args.steps):
            lad.replay_eager_step(cfg, S, S, *args_t(args.warmup + k), y)
        torch.cuda.synchronize()
        e1 = time.perf_counter()
        eager_out = {"value": B * args.steps / (e1 - e0), "unit": "tokens/s",
                     "ms_per_step": 1e3 * (e1 - e0) / args.steps,
                     "achieved_GBs": eager_bytes(w) * args.steps / (e1 - e0) / 1e9}
    del S
    torch.cuda.empty_cache()
    value = B * args.steps / elapsed
    out = {
        "metric": "Gated DeltaNet layer decode tokens/s at B=256 + achieved HBM GB/s (% peak) vs eager",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (seeded; unit-length q, k; {POOL_STEPS} distinct steps cycled)",
        "config": {"workload": "Gated DeltaNet layer, standard decode", "batch": B, "heads": H, "groups": G,
                   "head_dim": P, "state_dim": N, "ring_len": L, "io": "bf16", "checkpoint": "f32",
                   "read": args.read, "flush_every": L},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (_counter_traffic(GDN_SOURCES, "gdn_verify_kernel_f32_b256_h32_counters.txt")
                                 if read is None else None),
                     "kernel": "gdn_verify_kernel, W=1 (output-only: backward chain + one pass over S0)",
                     "avg_launch_us": 1e6 * dec_s / (reps * L), "timed_launches": reps * L,
                     "launches_from": f"{reps} windows (ring counts 1..{L}) as separate calls after the timed "
                                      "region, each output-only launch between HIP events",
                     "algorithmic_bytes_per_launch": dec_bytes / (reps * L),
                     "fold": {"avg_launch_us": 1e6 * fold_s / reps, "achieved": fold_bytes / fold_s / 1e9,
                              "frac": fold_bytes / fold_s / 1e9 / HBM_PEAK_GBS}},
        "eager": eager_out,
        "speedup_vs_eager": value / eager_out["value"] if eager_out else None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, rule="gdn")
    return out


# ---------------------------------------------------------------------------
def _events(n):
    import torch
    return [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]


def bench_verify(args):
    """Speculative verify: B=256, H=64, G=8, P=64, N=128, L=16, W=5 drafts per
    round (--window: up to 16), accepted drafts ~ Uniform{0..W}; each round =
    flush(L-W+1), append(W), verify(W) (one fused launch with --api step,
    three launches with --api calls or W > 8), then rollback(W - accepted)
    (with --api step that rollback rides on the next round's launch,
    replay_rollback_verify_step).
    The eager baseline drafts with W per-token steps into snapshots and
    restores the accepted one."""
    import torch
    import linear_attention_decode_amd as lad
    w = synth.named("verify")
    B, H, G, P, N, L, W = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len, args.window
    api = args.api if W <= 8 else "calls"   # windows past 8: flush, append and the matrix-core verify
    R = args.steps if args.steps_given else 128
    WU = args.warmup
    toks = input_pool(w, (R + WU) * W)
    acc_np = synth.accept_counts(w, R + WU, W)
    accept = torch.from_numpy(acc_np).cuda()
    nrej = (W - accept).to(torch.int32).contiguous()
    win = {k: v.view((R + WU), W, *v.shape[1:]).transpose(1, 2).contiguous() for k, v in toks.items()}
    rc = {"f32": None, "bf16": "bf16", "fp8": "fp8", "fp4": "fp4"}[args.read]
    st_bytes = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5}[args.read]
    layer = lad.ReplayLayer(B, H, G, P, N, L, io_dtype="bf16", read_copy=rc)
    y = torch.empty((B, W, H, P), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def round_(r, ev=None):
        drafts = (win["q"][r], win["k"][r], win["v"][r], win["dt"][r], win["a"][r])
        if api == "step":
            # one fused launch: the previous round's rollback, fold if due,
            # append the drafts, score them (this round's rollback rides on
            # the next launch; the last one is a plain rollback)
            if ev is not None:
                ev[0].record(stream)
            if r == 0:
                layer.verify_step(W, *drafts, y, flush_at=L - W + 1)
            else:
                layer.rollback_verify_step(nrej[r - 1], W, *drafts, y, flush_at=L - W + 1)
            if ev is not None:
                ev[1].record(stream)
            return
        else:
            layer.flush(L - W + 1)
            layer.append(W, *drafts)
            if ev is not None:
                ev[0].record(stream)
            layer.verify(W, y)
            if ev is not None:
                ev[1].record(stream)
        layer.rollback(nrej[r])

    for r in range(WU):
        round_(r)
    torch.cuda.synchronize()
    # HIP events bracket every stride-th round's launch (as in the decode
    # bench; folds here follow the random accept counts, not the round index)
    stride = args.event_stride or 4
    sampled = [k for k in range(R) if k % stride == 0]
    evs = dict(zip(sampled, _events(len(sampled))))
    t0 = time.perf_counter()
    for k in range(R):
        round_(WU + k, evs.get(k))
    if api == "step":
        layer.rollback(nrej[WU + R - 1])   # the last round's rollback, inside the timed region
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    assert layer.get_error()[0] == 0
    ver_ms = [evs[k][0].elapsed_time(evs[k][1]) for k in sampled]
    # ring counts at the start of every round and at verify time (host side)
    before, at_verify = _verify_counts(B, L, W, acc_np)
    if api == "step" and rc is not None:
        vbytes = sum(verify_step_copy_bytes(w, before[WU + k], W, st_bytes) for k in sampled)
        kernel_name = f"verify round, {args.read} read copy (fold + copy rewrite if due, append, verify; W={W})"
    elif api == "step":
        vbytes = sum(verify_step_bytes(w, before[WU + k], W) for k in sampled)
        kernel_name = f"verify round (fold if due + append + verify, W={W})"
    else:
        vbytes = sum(float(np.mean([decode_bytes(w, c, W, st_bytes) / B for c in at_verify[WU + k]])) * B
                     for k in sampled)
        kernel_name = f"verify (W={W}{', matrix cores' if W >= 6 else ''})"
    achieved = vbytes / (sum(ver_ms) / 1e3) / 1e9
    layer.close()
    del layer
    torch.cuda.empty_cache()

    # eager: W per-token steps into snapshots, then restore the accepted one
    eel = None
    if not args.no_eager:
        cfg = lad.ReplayConfig(B, H, G, P, N, L, lad.BF16, lad.NONE, 0)
        S = torch.zeros((B, H, P, N), dtype=torch.float32, device="cuda")
        snaps = torch.empty((W, B, H, P, N), dtype=torch.float32, device="cuda")
        ye = torch.empty((B, H, P), dtype=torch.float32, device="cuda")

        def eround(r):
            for i in range(W):
                t = r * W + i
                lad.replay_eager_step(cfg, S if i == 0 else snaps[i - 1], snaps[i], toks["q"][t], toks["k"][t],
                                      toks["v"][t], toks["dt"][t], toks["a"][t], ye)
            lad.replay_eager_select(cfg, snaps, W, accept[r], S)
        for r in range(WU):
            eround(r)
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        for k in range(R):
            eround(WU + k)
        torch.cuda.synchronize()
        eel = time.perf_counter() - e0
    acc_total = float(acc_np[WU:].sum())
    replay_round_bytes = (state_bytes(w) + B * (W * (H * P * 2 + H * 8 + 2 * G * N * 2)) * 2
                          + vbytes / len(sampled))
    eager_round_bytes = W * eager_bytes(w) + float(np.mean(acc_np[WU:] >= 1)) * 2 * state_bytes(w)
    return {
        "metric": "speculative verify: scored draft positions/s at B=256",
        "value": B * W * R / el, "unit": "positions/s", "n_gpus": 1, "steps": R, "warmup": WU,
        "ms_per_step": 1e3 * el / R, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": f"synthetic (seeded), accepted drafts ~ Uniform{{0..{W}}}",
        "config": {"workload": "speculative verify, one SSM layer", "batch": B, "heads": H, "groups": G,
                   "head_dim": P, "state_dim": N, "ring_len": L, "window": W, "rounds": R, "api": api,
                   "read_copy": args.read},
        "accepted_tokens_per_s": acc_total / el,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (_counter_traffic(VERIFY_STEP_SOURCES, "verify_step_kernel_b256_h64_w5_counters.txt")
                                 if api == "step" and W == 5 and rc is None else
                                 _counter_traffic(VERIFY_WIDE_SOURCES, "verify_wide_kernel_b256_h64_w16_counters.txt")
                                 if W == 16 else None),
                     "kernel": kernel_name,
                     "avg_launch_us": 1e3 * sum(ver_ms) / len(ver_ms),
                     "algorithmic_bytes_per_launch": vbytes / len(sampled), "timed_launches": len(sampled)},
        "eager": ({"positions_per_s": B * W * R / eel, "accepted_tokens_per_s": acc_total / eel,
                   "ms_per_round": 1e3 * eel / R} if eel else None),
        "speedup_vs_eager": eel / el if eel else None,
        "round_bytes_ratio_vs_eager": replay_round_bytes / eager_round_bytes,
    }


def _verify_counts(B, L, W, acc):
    """Ring counts of every round and sequence, at the round's start and at
    verify time: each round folds a ring holding at least L-W+1 entries,
    appends W drafts, verifies, then drops the W - accepted rejected drafts."""
    c = np.zeros(B, dtype=np.int64)
    before, at_verify = [], []
    for r in range(acc.shape[0]):
        before.append(c.copy())
        c = np.where(c >= L - W + 1, 0, c) + W
        at_verify.append(c.copy())
        c = c - (W - acc[r])
    return before, at_verify


def _tok_err(y, ref):
    """Per token: max over heads x P of |y - ref|, over max |ref|."""
    d = (y.double() - ref.double()).abs().amax(dim=(-2, -1))
    return d / ref.double().abs().amax(dim=(-2, -1)).clamp_min(1e-300)


def bench_dual(args):
    """Dual precision: decode shapes, T=1024 steps per mode; float32 master
    with reads from the master, a bf16 copy or an e4m3 copy (separated), and
    the shared low-precision checkpoint.  Each mode's outputs on sampled
    sequences are compared with the float32-master path's outputs per window
    (the float64 oracle comparison lives in the tests)."""
    import torch
    import linear_attention_decode_amd as lad
    T = args.steps if args.steps_given else 1024
    out_modes = {}
    for dt_scale in ([1.0, 0.01] if not args.quick else [1.0]):
        w = synth.named("dual", dt_scale=dt_scale)
        B, H, G, P, N, L = w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len
        seqs = [0, 101, 202]
        chunk = 128
        pools = [input_pool(w, chunk, t0=c0) for c0 in range(0, T, chunk)]
        ys_master = None
        for mode, rc, shared in [("f32", None, False), ("bf16-separated", "bf16", False),
                                 ("fp8-separated", "fp8", False), ("fp4-separated", "fp4", False),
                                 ("bf16-shared", "bf16", True), ("fp8-shared", "fp8", True),
                                 ("fp4-shared", "fp4", True)]:
            y = torch.empty((B, H, P), dtype=torch.float32, device="cuda")
            sel = torch.tensor(seqs, device="cuda")

            def run(capture):
                layer = lad.ReplayLayer(B, H, G, P, N, L, io_dtype="bf16", read_copy=rc, shared_lowp=shared)
                ys = torch.empty((T, len(seqs), H, P), dtype=torch.float32, device="cuda")
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for t in range(T):
                    p = pools[t // chunk]
                    i = t % chunk
                    layer.step(p["q"][i], p["k"][i], p["v"][i], p["dt"][i], p["a"][i], y, flush_at=L)
                    if capture:
                        ys[t] = y.index_select(0, sel)
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
                assert layer.get_error()[0] == 0
                layer.close()
                return el, ys
            _, ys = run(True)           # pass that keeps the sampled outputs (also the warm-up)
            el, _ = run(False)          # timed pass
            key = mode if dt_scale == 1.0 else f"{mode} (dt x{dt_scale})"
            rec = {"tokens_per_s": B * T / el}
            if ys_master is None:
                ys_master = ys
            else:
                e_tok = _tok_err(ys, ys_master).cpu().numpy()               # [T][b]
                nw = T // L
                per_win = e_tok[: nw * L].reshape(nw, L, -1)
                rec.update({"max_err_vs_master": float(e_tok.max()), "mean_err_vs_master": float(e_tok.mean()),
                            "drift_max_mean": {f"window_{i}": [float(per_win[i].max()), float(per_win[i].mean())]
                                               for i in sorted({0, nw // 2, nw - 1})}})
            out_modes[key] = rec
            torch.cuda.empty_cache()
    first = out_modes["fp8-separated"]
    return {
        "metric": "dual-precision decode tokens/s at B=256 (+ error drift vs the float32 master path)",
        "value": first["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": T, "warmup": 0,
        "ms_per_step": 1e3 * 256 / first["tokens_per_s"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded)",
        "config": {"workload": "dual-precision decode, one SSM layer", "batch": 256, "heads": 128,
                   "groups": 8, "head_dim": 64, "state_dim": 128, "ring_len": 16, "steps": T,
                   "value_is": "fp8-separated", "error_metric": "per token, max|dy|/max|y| over heads x P"},
        "modes": out_modes,
    }


def bench_stacked(args):
    """Stacked sweep: 8 SSM layers, B=512, H=64, G=8, P=N=128, ring L in
    {8, 16, 32}; T=512 steps, each layer cycling 64 pre-generated steps of its
    own seeded inputs; ReplaySSM (fused step) against the eager per-token
    baseline."""
    import torch
    import linear_attention_decode_amd as lad
    T = args.steps if args.steps_given else 512
    pool_n = 64
    res = {}
    Ls = [8, 16, 32] if not args.quick else [16]
    pools = [input_pool(synth.named("stacked", layer=li), pool_n) for li in range(8)]
    for L in Ls:
        w = synth.named("stacked", ring_len=L)
        B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
        layers = [lad.ReplayLayer(B, H, G, P, N, L, io_dtype="bf16") for _ in range(8)]
        y = torch.empty((B, H, P), dtype=torch.float32, device="cuda")

        ys = [torch.empty((B, H, P), dtype=torch.float32, device="cuda") for _ in range(8)]

        def step(t):
            i = t % pool_n
            if args.api == "layers":
                # one launch steps all 8 layers
                lad.replay_step_layers([x.h for x in layers], [p["q"][i] for p in pools], [p["k"][i] for p in pools],
                                       [p["v"][i] for p in pools], [p["dt"][i] for p in pools],
                                       [p["a"][i] for p in pools], ys, L)
                return
            for li in range(8):
                p = pools[li]
                layers[li].step(p["q"][i], p["k"][i], p["v"][i], p["dt"][i], p["a"][i], y, flush_at=L)
        for t in range(L):
            step(t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(L, L + T):
            step(t)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        for lay in layers:
            assert lay.get_error()[0] == 0
            lay.close()
        del layers
        torch.cuda.empty_cache()
        window_replay = (sum(step_bytes(w, c, c >= L) for c in range(1, L + 1))) * 8
        window_eager = L * eager_bytes(w) * 8
        res[f"L={L}"] = {"tokens_per_s": B * T / el, "ms_per_step": 1e3 * el / T,
                         "window_bytes_ratio_vs_eager": window_replay / window_eager,
                         "achieved_GBs": window_replay / L * T / el / 1e9}
    # eager baseline (does not depend on L)
    w = synth.named("stacked")
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    cfg = lad.ReplayConfig(B, H, G, P, N, 16, lad.BF16, lad.NONE, 0)
    Ss = [torch.zeros((B, H, P, N), dtype=torch.float32, device="cuda") for _ in range(8)]
    y = torch.empty((B, H, P), dtype=torch.float32, device="cuda")

    def estep(t):
        i = t % pool_n
        for li in range(8):
            p = pools[li]
            lad.replay_eager_step(cfg, Ss[li], Ss[li], p["q"][i], p["k"][i], p["v"][i], p["dt"][i], p["a"][i], y)
    for t in range(8):
        estep(t)
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    Te = min(T, 128)
    for t in range(Te):
        estep(t)
    torch.cuda.synchronize()
    eel = time.perf_counter() - e0
    eager = {"tokens_per_s": B * Te / eel, "ms_per_step": 1e3 * eel / Te,
             "achieved_GBs": eager_bytes(w) * 8 * Te / eel / 1e9}
    best = max(res.values(), key=lambda r: r["tokens_per_s"])
    return {
        "metric": "8-layer stacked decode tokens/s at B=512 per ring length vs eager",
        "value": res.get("L=16", best)["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": T,
        "warmup": 0, "ms_per_step": res.get("L=16", best)["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (seeded, {pool_n} distinct steps per layer cycled)",
        "config": {"workload": "8 stacked SSM layers", "batch": 512, "heads": 64, "groups": 8,
                   "head_dim": 128, "state_dim": 128, "ring_len": "8/16/32", "value_is": "L=16",
                   "api": "one launch for all layers" if args.api == "layers" else "one launch per layer"},
        "per_ring_len": res, "eager": eager,
        "speedup_vs_eager_L16": res.get("L=16", best)["tokens_per_s"] / eager["tokens_per_s"],
    }


def bench_stacked_latency(args):
    """Stacked layers (8 layers, H=64, G=8, P=N=128, L=16) at batch 1, 16 and
    512: time per 8-layer decode step for the 8 per-layer launches
    (replay_step) and for the single launch over all layers
    (replay_step_layers), each issued eagerly and replayed from a HIP graph
    of one step (inputs copied into the captured buffers before each replay
    are not timed: the graph reads a pool slot the loop rotates)."""
    import torch
    import linear_attention_decode_amd as lad
    L, NL = 16, 8
    out = {}
    for B in args.batches:
        T = 32 if B >= 256 else (64 if B >= 64 else 256)
        ws = [synth.named("stacked", batch=B, layer=li) for li in range(NL)]
        w = ws[0]
        H, G, P, N = w.heads, w.groups, w.head_dim, w.state_dim
        pools = [input_pool(x, 16) for x in ws]
        res = {}
        for api in ("step", "layers"):
            for graphed in (False, True):
                layers = [lad.ReplayLayer(B, H, G, P, N, L, io_dtype="bf16") for _ in range(NL)]
                y = [torch.empty((B, H, P), dtype=torch.float32, device="cuda") for _ in range(NL)]
                slot = [{k: v[0].clone() for k, v in p.items()} for p in pools]

                def one(src):
                    if api == "step":
                        for li in range(NL):
                            layers[li].step(src[li]["q"], src[li]["k"], src[li]["v"], src[li]["dt"], src[li]["a"],
                                            y[li], flush_at=L)
                    else:
                        lad.replay_step_layers([x.h for x in layers], [src[li]["q"] for li in range(NL)],
                                               [src[li]["k"] for li in range(NL)], [src[li]["v"] for li in range(NL)],
                                               [src[li]["dt"] for li in range(NL)], [src[li]["a"] for li in range(NL)],
                                               y, L)
                pool_t = lambda t: [{k: v[t % 16] for k, v in p.items()} for p in pools]
                for t in range(L):          # warm up one window
                    one(pool_t(t))
                torch.cuda.synchronize()
                if graphed:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        one(slot)
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    for t in range(T):
                        g.replay()
                    torch.cuda.synchronize()
                else:
                    t0 = time.perf_counter()
                    for t in range(T):
                        one(pool_t(t))
                    torch.cuda.synchronize()
                el = time.perf_counter() - t0
                for x in layers:
                    assert x.get_error()[0] == 0
                    x.close()
                del layers
                torch.cuda.empty_cache()
                res[f"{api}{'-graph' if graphed else ''}"] = 1e6 * el / T
        res["tokens_per_s_best"] = B * 1e6 / min(v for k, v in res.items())
        out[f"B={B}"] = res
    return {
        "metric": "8-layer stacked decode step time (us) by launch form, per batch",
        "value": out[f"B={args.batches[0]}"]["layers-graph"], "unit": "us per 8-layer step", "n_gpus": 1,
        "steps": None, "warmup": 16, "ms_per_step": out[f"B={args.batches[0]}"]["layers-graph"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded, 16 steps per layer cycled)",
        "config": {"workload": "8 stacked SSM layers, step latency", "heads": 64, "groups": 8, "head_dim": 128,
                   "state_dim": 128, "ring_len": L,
                   "value_is": f"B={args.batches[0]}, one launch for all layers, graph"},
        "us_per_step": out,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="decode", choices=["decode", "verify", "dual", "stacked", "stacked-latency",
                                                             "gdn"])
    ap.add_argument("--quick", action="store_true", help="dual/stacked: one variant only")
    ap.add_argument("--window", type=int, default=5,
                    help="verify: drafts per round (5 is the benchmarked workload; up to 16, windows past 8 "
                         "on the matrix cores through the separate calls)")
    ap.add_argument("--api", default="step", choices=["step", "calls", "layers"],
                    help="step: one fused launch per decode step (replay_step) or verify round "
                         "(replay_verify_step); calls: the append, decode/verify and flush kernels; "
                         "layers (stacked): one launch steps all layers (replay_step_layers)")
    ap.add_argument("--read", default="f32", choices=["f32", "bf16", "fp8", "fp4"],
                    help="checkpoint the outputs read: the float32 master or a bf16 / e4m3 / MX FP4 copy")
    ap.add_argument("--event-stride", type=int, default=0,
                    help="verify: bracket every n-th round's launch with HIP events (default 4)")
    ap.add_argument("--roofline-windows", type=int, default=4,
                    help="decode: whole windows run back to back after the timed region for the roofline")
    ap.add_argument("--batches", type=lambda t: [int(x) for x in t.split(",")], default=[1, 16, 512],
                    help="stacked-latency: batch sizes, comma-separated")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eager", action="store_true", help="skip the eager baseline timing")
    ap.add_argument("--probe-copy-gib", type=float, default=0.0,
                    help="first run the plain copy probe over this many GiB (counter calibration)")
    args = ap.parse_args()
    args.steps_given = any(a.startswith("--steps") for a in sys.argv[1:])
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU (the decode path needs no collective); --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.probe_copy_gib > 0:
        import linear_attention_decode_amd as lad
        nbytes = int(args.probe_copy_gib * (1 << 30)) // 16 * 16
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        lad.replay_stream_probe(1, src, dst, nbytes)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    # The decode workload reports its kernel against the chip's measured read
    # ceiling.  That probe runs first, before the layer is built: the timed
    # steps then start on a GPU that has been streaming for some milliseconds,
    # as it is in service, instead of paying the clocks' ramp from idle
    # (about 4 us a step over the first hundred steps of a cold start).
    args.read_ceiling = read_ceiling_gbs() if args.workload == "decode" else None
    out = {"decode": bench_decode, "verify": bench_verify, "dual": bench_dual,
           "stacked": bench_stacked, "stacked-latency": bench_stacked_latency, "gdn": bench_gdn}[args.workload](args)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
