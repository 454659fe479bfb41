"""The parity metric for outputs read from a float32 checkpoint (numpy only).

The stated bound is a maximum relative error of 1e-4, taken per head:
rel(b, t, h) = max_p |y - y_ref| / max_p |y_ref| against the float64 oracle.
Its denominator is floored at COND_FLOOR times the head's term magnitude
max_p y_abs, where y_abs is the same recurrence run on |q|, |k|, |v| (dt and
a are positive): the sum of the absolute values of every product that makes
up y.  The floor matters only for a head whose output cancels by more than
1 / COND_FLOOR against its own terms, typically where k . q is close to
zero.  There no float32 evaluation can hold 1e-4 of the output, the plain
definition's included (tests/test_parity_metric.py pins this), and the
bound becomes 1e-4 * COND_FLOOR = 1e-6 of the term magnitude, about 17
units of float32 rounding (2^-24).  A fault that changes a term (a wrong
decay, slot, group or head index) moves y by a sizable fraction of y_abs
and still fails it.
"""
from __future__ import annotations

import numpy as np

TOL_F32 = 1e-4
COND_FLOOR = 1e-2


def abs_inputs(x: dict) -> dict:
    """float64 oracle inputs with q, k, v replaced by their absolute values."""
    return {k: (np.abs(v) if k in ("q", "k", "v") else v) for k, v in x.items()}


def per_head_errors(y: np.ndarray, y_ref: np.ndarray, y_abs: np.ndarray):
    """(floored per-head error, plain per-head error) arrays over [..][H];
    inputs end in [..][H][P]."""
    num = np.max(np.abs(np.asarray(y, dtype=np.float64) - y_ref), axis=-1)
    den = np.max(np.abs(y_ref), axis=-1)
    mag = np.max(np.asarray(y_abs, dtype=np.float64), axis=-1)
    floored = num / np.maximum(np.maximum(den, COND_FLOOR * mag), 1e-30)
    plain = num / np.maximum(den, 1e-30)
    return floored, plain


def per_token_error(y: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """max over (heads, P) of |y - y_ref| over max |y_ref|: one token's layer output."""
    num = np.max(np.abs(np.asarray(y, dtype=np.float64) - y_ref), axis=(-2, -1))
    return num / np.maximum(np.max(np.abs(y_ref), axis=(-2, -1)), 1e-30)
