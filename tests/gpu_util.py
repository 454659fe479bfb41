"""Helpers for the GPU parity tests: move seeded inputs to the device, drive
the C ABI through the Python binding, and keep the integer ring model in
step with every call."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import ring as oring
from oracle import runs
from tests import parity

DEV = torch.device("cuda:0")


def note(msg: str):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, io_dtype: str | None = None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


class DevInputs:
    """Seeded inputs of tokens [t0, t1) for all sequences, on the device:
    q, k [T][B][G][N], v [T][B][H][P], dt, a [T][B][H]."""

    def __init__(self, w: synth.Workload, t0: int, t1: int):
        self.w = w
        self.t0 = t0
        inp = synth.step_inputs(w, t0, t1)
        self.t = {k: to_dev(v) for k, v in inp.items()}

    def step(self, t: int):
        i = t - self.t0
        return tuple(self.t[n][i] for n in ("q", "k", "v", "dt", "a"))

    def window(self, t: int, W: int):
        """Tokens t..t+W-1 as [B][W][...] tensors (the append layout)."""
        i = t - self.t0
        return tuple(self.t[n][i:i + W].transpose(0, 1).contiguous() for n in ("q", "k", "v", "dt", "a"))


class DevInputsTorch(DevInputs):
    """As DevInputs, generated on the device (synth.step_inputs_torch) for
    full-batch runs; the oracle is fed the very bytes the device holds."""

    def __init__(self, w: synth.Workload, t0: int, t1: int):
        self.w = w
        self.t0 = t0
        self.t = synth.step_inputs_torch(w, t0, t1, device=DEV)

    def oracle(self, seqs=None) -> dict:
        """float64 oracle inputs [T][b][...] of sequences `seqs` (all if None)."""
        pick = (lambda v: v) if seqs is None else (lambda v: v[:, seqs])
        return runs.widen_inputs({k: synth.to_storage(pick(v)) for k, v in self.t.items()}, self.w.io_dtype)


def oracle_inputs(w: synth.Workload, t0: int, t1: int, seqs) -> dict:
    return runs.widen_inputs(synth.step_inputs(w, t0, t1, seqs=seqs), w.io_dtype)


def check_ring(layer, model: oring.RingModel, what: str):
    pos = layer.pos.cpu().numpy()
    base = layer.base.cpu().numpy()
    assert np.array_equal(pos, model.pos), f"pos differs after {what}"
    assert np.array_equal(base, model.base), f"base differs after {what}"


def run_standard(layer, w: synth.Workload, dev: DevInputs, t0: int, t1: int, model=None,
                 y_out: torch.Tensor | None = None):
    """append(1); decode; flush(L) per step.  Returns y [T][B][H][P] (device)."""
    B, H, P, L = w.batch, w.heads, w.head_dim, w.ring_len
    y = y_out if y_out is not None else torch.empty((t1 - t0, B, H, P), dtype=torch.float32, device=DEV)
    for t in range(t0, t1):
        q, k, v, dt, a = dev.step(t)
        layer.append(1, q, k, v, dt, a)
        layer.decode(y[t - t0])
        layer.flush(L)
        if model is not None:
            model.append(1)
            model.read(1)
            model.flush(L)
            check_ring(layer, model, f"step {t}")
    return y


def errors(y_gpu: np.ndarray, y_ref: np.ndarray):
    """(max per-token error over the layer output, max per-head-vector error,
    mean per-head-vector error)."""
    e_tok = runs.normwise_rel_err(y_gpu, y_ref)
    e_vec = runs.normwise_rel_err(y_gpu, y_ref, axes=(-1,))
    return float(np.max(e_tok)), float(np.max(e_vec)), float(np.mean(e_vec))


TOL_F32 = parity.TOL_F32


# Outputs read from a low-precision copy against the oracle's emulation of
# the same copy (built from the float64 state rounded to float32).  The
# device's float32 master differs from that state by float32 rounding, and
# where a value sits that close to a code boundary the two round to
# neighbouring codes: sparse outliers of up to 1.8e-3 per token were measured
# for e4m3 and FP4 (speculative rounds at B=256, H=64, W=5, 16 sequences x
# 32 rounds: 25 and 10 of 2560 outputs above 1e-4, all others at 2e-7), so
# the maximum is bounded at 5e-3 (1e-3 for bf16, whose codes are 8 times
# finer), and the median, which a systematic error would move, at 1e-6.
COPY_TOL_MAX = {"bf16": 1e-3, "fp8": 5e-3, "fp4": 5e-3}
COPY_TOL_MEDIAN = 1e-6


def assert_copy(y_gpu: np.ndarray, y_emul: np.ndarray, fmt: str, what: str = ""):
    """Per-token error against the emulation of the same copy: max and median bounds."""
    e = runs.normwise_rel_err(y_gpu, y_emul)
    mx, med = float(np.max(e)), float(np.median(e))
    print(f"  {what} vs emulation of the {fmt} copy: per-token max {mx:.3e} median {med:.3e}", flush=True)
    assert mx <= COPY_TOL_MAX[fmt], f"{what} {fmt}: max {mx:.3e} > {COPY_TOL_MAX[fmt]:.0e}"
    assert med <= COPY_TOL_MEDIAN, f"{what} {fmt}: median {med:.3e} > {COPY_TOL_MEDIAN:.0e}"
    return mx


def y_abs_standard(x: dict, S_shape) -> np.ndarray:
    """Term magnitudes of standard decode from a zero state: the oracle on |q|, |k|, |v|."""
    return runs.standard(parity.abs_inputs(x), np.zeros(S_shape))


def y_abs_verify(x: dict, accept: np.ndarray, W: int, S_shape) -> np.ndarray:
    """Term magnitudes of speculative rounds from a zero state ([R][W][B][H][P])."""
    return runs.verify_rounds(parity.abs_inputs(x), accept, W, np.zeros(S_shape))


def assert_f32(y_gpu: np.ndarray, y_ref: np.ndarray, y_abs: np.ndarray, tol: float = TOL_F32, what: str = ""):
    """Parity of outputs read from a float32 checkpoint against the float64
    oracle (tests/parity.py): the per-head error max_p |y - y_ref| / max_p
    |y_ref|, its denominator floored at 1 % of the head's term magnitude
    max_p y_abs, must not exceed `tol` (1e-4) for any (sequence, token,
    head), and the per-token error over the layer's whole output must not
    either.  y arrays end in [..][H][P]; y_abs is the oracle's output on |q|,
    |k|, |v| (parity.abs_inputs)."""
    floored, plain = parity.per_head_errors(y_gpu, y_ref, y_abs)
    tok = float(np.max(parity.per_token_error(y_gpu, y_ref)))
    cond = np.max(np.abs(y_ref), axis=-1) / np.maximum(np.max(y_abs, axis=-1), 1e-300)
    n_floor = int(np.sum(cond < parity.COND_FLOOR))
    print(f"  {what} per-head max {floored.max():.3e} (without the floor {plain.max():.3e}; floor active on "
          f"{n_floor} of {floored.size} heads) mean {floored.mean():.3e}; per-token max {tok:.3e}", flush=True)
    assert floored.max() <= tol, f"{what} per-head error {floored.max():.3e} > {tol:.0e}"
    assert tok <= tol, f"{what} per-token error {tok:.3e} > {tol:.0e}"
    return tok, float(floored.max())


def run_verify(layer, w: synth.Workload, dev: DevInputs, R: int, W: int, accept: np.ndarray, model=None,
               fused: bool = False, rollback_fused: bool = False, nrej=None):
    """Speculative rounds: flush(L-W+1); append(W drafts); verify(W) -- as
    three calls, or as one replay_verify_step with fused=True -- then
    rollback(W - accepted).  Round r drafts tokens rW..rW+W-1.  With
    rollback_fused=True round r > 0 is one replay_rollback_verify_step
    carrying round r-1's rollback, and a plain rollback ends the run.
    nrej (int32 [R][B]) overrides the rejected counts W - accept.
    Returns y [R][B][W][H][P] (device)."""
    B, H, P, L = w.batch, w.heads, w.head_dim, w.ring_len
    y = torch.empty((R, B, W, H, P), dtype=torch.float32, device=DEV)
    nrej_np = (W - accept).astype(np.int32) if nrej is None else np.asarray(nrej, dtype=np.int32)
    nrej = torch.from_numpy(nrej_np).to(DEV)
    if rollback_fused:
        for rd in range(R):
            if rd == 0:
                layer.verify_step(W, *dev.window(0, W), y[0], flush_at=L - W + 1)
            else:
                layer.rollback_verify_step(nrej[rd - 1], W, *dev.window(rd * W, W), y[rd], flush_at=L - W + 1)
            if model is not None:
                if rd > 0:
                    model.rollback(nrej_np[rd - 1])
                model.flush(L - W + 1)
                model.append(W)
                model.read(W)
                check_ring(layer, model, f"round {rd}")
        layer.rollback(nrej[R - 1])
        if model is not None:
            model.rollback(nrej_np[R - 1])
            check_ring(layer, model, "last rollback")
        return y
    for rd in range(R):
        if fused:
            layer.verify_step(W, *dev.window(rd * W, W), y[rd], flush_at=L - W + 1)
        else:
            layer.flush(L - W + 1)
            layer.append(W, *dev.window(rd * W, W))
            layer.verify(W, y[rd])
        layer.rollback(nrej[rd])
        if model is not None:
            model.flush(L - W + 1)
            model.append(W)
            model.read(W)
            model.rollback(nrej_np[rd])
            check_ring(layer, model, f"round {rd}")
    return y
