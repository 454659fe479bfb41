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
    """(max per-token error over the layer output, max per-head-vector error)."""
    e_tok = runs.normwise_rel_err(y_gpu, y_ref)
    e_vec = runs.normwise_rel_err(y_gpu, y_ref, axes=(-1,))
    return float(np.max(e_tok)), float(np.max(e_vec)), float(np.mean(e_vec))


def run_verify(layer, w: synth.Workload, dev: DevInputs, R: int, W: int, accept: np.ndarray, model=None,
               fused: bool = False):
    """Speculative rounds: flush(L-W+1); append(W drafts); verify(W) -- as
    three calls, or as one replay_verify_step with fused=True -- then
    rollback(W - accepted).  Round r drafts tokens rW..rW+W-1.
    Returns y [R][B][W][H][P] (device)."""
    B, H, P, L = w.batch, w.heads, w.head_dim, w.ring_len
    y = torch.empty((R, B, W, H, P), dtype=torch.float32, device=DEV)
    nrej = torch.from_numpy((W - accept).astype(np.int32)).to(DEV)
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
            model.rollback(W - accept[rd])
            check_ring(layer, model, f"round {rd}")
    return y
