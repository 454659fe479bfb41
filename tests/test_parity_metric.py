"""Pins of the float32 parity metric (tests/parity.py), CPU only.

1. The plain per-head bound cannot be met by float32 arithmetic: the pages'
   eager recurrence (page "ReplaySSM: Cachear Inputs, No Estado", eq.
   "Forma resumen") evaluated in float32, with every product and every
   running sum rounded in order, misses 1e-4 per head on the decode
   recipe's first tokens of sequence 144, where the group's k . q cancels
   (the output is about 5000x smaller than its terms).  The floored metric
   accepts it with a wide margin.
2. The floor does not hide faults: planted mistakes confined to one head of
   one sequence (a decay taken from the neighbouring head, a dropped dt, a
   head whose output is zeroed -- the lowest-magnitude one) fail it.
"""
import numpy as np
import pytest

import synth
from oracle import runs
from tests import parity

SEQ, T = 144, 4


@pytest.fixture(scope="module")
def case():
    w = synth.named("decode")
    x = runs.widen_inputs(synth.step_inputs(w, 0, T, seqs=[SEQ]), w.io_dtype)
    S = np.zeros((1, w.heads, w.head_dim, w.state_dim))
    y_ref = runs.standard(x, S.copy())
    y_abs = runs.standard(parity.abs_inputs(x), S.copy())
    return w, x, y_ref, y_abs


def _eager_f32(w, x, fault=None, head=8):
    """The eager recurrence in float32: S <- a S + dt v k^T, y = S q, the
    dot products summed in order (np.cumsum is sequential)."""
    G, H = w.groups, w.heads
    g = np.arange(H) * G // H
    S = np.zeros((1, H, w.head_dim, w.state_dim), np.float32)
    ys = []
    for t in range(T):
        q = x["q"][t].astype(np.float32)[:, g]
        k = x["k"][t].astype(np.float32)[:, g]
        v = x["v"][t].astype(np.float32)
        dt = x["dt"][t].astype(np.float32).copy()
        a = x["a"][t].astype(np.float32).copy()
        if fault == "decay of the next head":
            a[:, head] = a[:, head + 1]
        if fault == "dropped dt":
            dt[:, head] = 1.0
        S = (a[..., None, None] * S + (dt[..., None] * v)[..., None] * k[..., None, :]).astype(np.float32)
        y = np.cumsum(S * q[:, :, None, :], axis=-1, dtype=np.float32)[..., -1]
        ys.append(y)
    return np.stack(ys)


def test_float32_definition_needs_the_floor(case):
    w, x, y_ref, y_abs = case
    floored, plain = parity.per_head_errors(_eager_f32(w, x), y_ref, y_abs)
    cond = np.max(np.abs(y_ref), -1) / np.max(y_abs, -1)
    assert plain.max() > parity.TOL_F32, plain.max()          # the plain bound is out of reach
    assert cond[plain > parity.TOL_F32].max() < 1e-3           # ... only on heads that cancel
    assert floored.max() < 0.1 * parity.TOL_F32, floored.max()
    assert parity.per_token_error(_eager_f32(w, x), y_ref).max() < 1e-5


@pytest.mark.parametrize("fault", ["decay of the next head", "dropped dt"])
def test_floor_keeps_faults_visible(case, fault):
    w, x, y_ref, y_abs = case
    floored, _ = parity.per_head_errors(_eager_f32(w, x, fault), y_ref, y_abs)
    assert floored.max() > 100 * parity.TOL_F32, (fault, floored.max())


def test_zeroed_low_magnitude_head_is_caught(case):
    w, x, y_ref, y_abs = case
    y = _eager_f32(w, x)
    mag = np.max(np.abs(y_ref), -1)
    t, b, h = np.unravel_index(np.argmin(mag), mag.shape)
    y[t, b, h] = 0.0
    floored, _ = parity.per_head_errors(y, y_ref, y_abs)
    assert floored[t, b, h] > parity.TOL_F32
