"""Benchmark of the ReplaySSM decode path on one MI355X.

Default workload (the headline): one Mamba-2-shaped SSM layer in standard
decode -- batch 256, 128 heads, 8 groups, P=64, N=128, ring L=16, bf16
q/k/v, float32 checkpoint.  One step = append one token per sequence, the
output-only decode of that token, and the flush of every ring that became
full (every 16th step).  The timed region is K steps (default 256 = 16
windows) with all inputs resident in HBM; the eager per-token baseline is
timed the same way on the same inputs.

Prints ONE JSON line.  `roofline` is the decode kernel (the dominant one):
algorithmic bytes per launch / its average duration from HIP events on the
launch stream.  `cpu_baseline` is the float64 oracle on a bounded sample of
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
    return w.batch * w.heads * w.head_dim * w.state_dim * st_bytes


def decode_bytes(w, count, W=1, st_bytes=4, io=2):
    """One decode/verify launch with `count` live entries per sequence."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io          # v, (dt, a), k
    scale = H * 4 if st_bytes == 1 else 0
    return (state_bytes(w, st_bytes) + scale
            + B * (count * per_entry + W * G * N * io + W * H * P * 4))   # + q + y


def flush_bytes(w, count, copy_bytes=0, io=2):
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io
    s = state_bytes(w)
    return 2 * s + B * count * per_entry + (state_bytes(w, copy_bytes) if copy_bytes else 0) \
        + (B * H * 4 if copy_bytes == 1 else 0)


def step_bytes(w, count, fold, io=2):
    """One fused step launch; `count` includes this step's token, which is read
    from the inputs and written to the ring."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    per_entry = H * P * io + H * 8 + G * N * io
    token = H * P * io + H * 8 + 2 * G * N * io          # v, (dt, a), q, k of the new token
    return (state_bytes(w) * (2 if fold else 1)
            + B * ((count - 1) * per_entry + 2 * token + H * P * 4))


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


def input_pool(w, nsteps):
    """nsteps seeded steps, resident on the device: q,k [T][B][G][N] ..."""
    inp = synth.step_inputs(w, 0, nsteps)
    return {k: _dev(v) for k, v in inp.items()}


def cpu_baseline(w, target_s=12.0, steps=256, chunk=32):
    """The oracle, as it stands, on a bounded sample of the workload: the
    first `nseq` sequences over all `steps` decode steps, nseq chosen from a
    short calibration so the sample takes about target_s seconds of host
    time.  Inputs are generated chunk by chunk outside the timed calls."""
    import oracle
    from oracle import runs

    def run(nseq, T, S):
        total = 0.0
        for t0 in range(0, T, chunk):
            x = runs.widen_inputs(synth.step_inputs(w, t0, min(T, t0 + chunk), seqs=list(range(nseq))),
                                  w.io_dtype)
            c0 = time.perf_counter()
            runs.standard(x, S)
            total += time.perf_counter() - c0
        return total

    cal_seq, cal_T = 4, 32
    cal = run(cal_seq, cal_T, np.zeros((cal_seq, w.heads, w.head_dim, w.state_dim)))
    per_token = cal / (cal_seq * cal_T)
    nseq = int(max(4, min(w.batch, target_s / (per_token * steps))))
    S = np.zeros((nseq, w.heads, w.head_dim, w.state_dim))
    dt = run(nseq, steps, S)
    return {"value": nseq * steps / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"float64 eager recurrence, first {nseq} of {w.batch} sequences x {steps} steps "
                      f"of the same layer ({dt:.1f} s host time, input generation excluded)"}


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
                  "linear_attention_decode_amd/csrc/device_common.h"]
STEP_SOURCES = ["linear_attention_decode_amd/csrc/step.hip",
                "linear_attention_decode_amd/csrc/device_common.h"]


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
    rc = {"f32": None, "bf16": "bf16", "fp8": "fp8"}[args.read]
    st_bytes = {"f32": 4, "bf16": 2, "fp8": 1}[args.read]
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    word, _ = layer.get_error()
    assert word == 0, f"device error bits {word}"
    elapsed = t1 - t0
    counts = [((args.warmup + k) % L) + 1 for k in range(args.steps)]
    if args.api == "step":
        # the dominant kernel is the fused step kernel itself
        step_ms = [e[0].elapsed_time(e[1]) for e in evs]
        folds = [c >= L for c in counts]
        dec_ms = [m for m, f in zip(step_ms, folds) if not f]
        fl_ms = [m for m, f in zip(step_ms, folds) if f]
        kernel_bytes = sum(step_bytes(w, c, c >= L) for c in counts)
        kernel_time = sum(step_ms) / 1e3
        avg_us = 1e3 * sum(step_ms) / len(step_ms)
        kernel_name = "step (append + output-only decode, or append + fold on full rings)"
    else:
        dec_ms = [e[0].elapsed_time(e[1]) for e in evs]
        fl_ms = [evs[k][2].elapsed_time(evs[k][3]) for k in range(args.steps) if (args.warmup + k + 1) % L == 0]
        kernel_bytes = sum(decode_bytes(w, c, 1, st_bytes) for c in counts)
        kernel_time = sum(dec_ms) / 1e3
        avg_us = 1e3 * sum(dec_ms) / len(dec_ms)
        kernel_name = "decode (output-only)"
    achieved = kernel_bytes / kernel_time / 1e9
    layer.close()
    del layer
    torch.cuda.empty_cache()

    eager_out = None if args.no_eager else _bench_eager(args, w, pool, y)

    window_replay = sum(decode_bytes(w, c, 1, st_bytes) for c in range(1, L + 1)) \
        + flush_bytes(w, L, 0 if st_bytes == 4 else st_bytes) \
        + B * L * 2 * (H * P * 2 + H * 8 + 2 * G * N * 2)            # appends: read input + write ring
    window_eager = L * eager_bytes(w)
    if args.api == "step":
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
                     "kernel": kernel_name, "avg_launch_us": avg_us,
                     "algorithmic_bytes_per_launch": kernel_bytes / len(counts)},
        "decode_avg_us": 1e3 * sum(dec_ms) / max(1, len(dec_ms)),
        "flush_avg_us": 1e3 * sum(fl_ms) / max(1, len(fl_ms)),
        "eager": eager_out,
        "speedup_vs_eager": (B * args.steps / elapsed) / eager_out["value"] if eager_out else None,
        "window_bytes_ratio_vs_eager": window_replay / window_eager,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="decode", choices=["decode"])
    ap.add_argument("--api", default="step", choices=["step", "calls"],
                    help="step: one fused replay_step launch per step; calls: append, decode, flush")
    ap.add_argument("--read", default="f32", choices=["f32", "bf16", "fp8"],
                    help="checkpoint the outputs read: the float32 master or a bf16 / e4m3 copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eager", action="store_true", help="skip the eager baseline timing")
    ap.add_argument("--probe-copy-gib", type=float, default=0.0,
                    help="first run the plain copy probe over this many GiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path needs no collective and this build runs "
              "on a single MI355X; --gpus must be 1", file=sys.stderr)
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
    out = bench_decode(args)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
