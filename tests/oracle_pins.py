"""Pins of the float64 eager oracle against things other than itself.

Each check takes ``eager_fn(S, q, k, v, dt, a) -> y`` (the signature of
``oracle.core.eager``) so the same checks run against deliberately broken
builds of the oracle (tests/test_oracle_pins.py plants mistakes in a copy of
its C source and requires at least one check to fail for each).

Every check returns None on success and raises AssertionError otherwise.
"""
from __future__ import annotations

import os

import numpy as np

from oracle import forms

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(rng, T, B, H, G, P, N, decay="rand"):
    q = rng.standard_normal((T, B, G, N))
    k = rng.standard_normal((T, B, G, N))
    v = rng.standard_normal((T, B, H, P))
    dt = rng.uniform(0.1, 2.0, (T, B, H))
    if decay == "rand":
        a = rng.uniform(0.2, 0.99, (T, B, H))
    else:
        a = np.full((T, B, H), float(decay))
    return q, k, v, dt, a


def _states(eager_fn, S, q, k, v, dt, a):
    """State after every token, via T one-token calls."""
    out = []
    ys = []
    for t in range(q.shape[0]):
        ys.append(eager_fn(S, q[t:t + 1], k[t:t + 1], v[t:t + 1], dt[t:t + 1], a[t:t + 1])[0])
        out.append(S.copy())
    return np.stack(out), np.stack(ys)


def _close(x, ref, tol=1e-12):
    scale = max(np.max(np.abs(ref)), 1e-300)
    err = np.max(np.abs(x - ref)) / scale
    assert err <= tol, f"relative error {err:.3e} > {tol:.1e}"


def check_history_form(eager_fn, seed=1):
    """Zero initial state: eager states equal eq. "Forma historia"."""
    rng = np.random.default_rng(seed)
    T, P, N = 7, 3, 5
    q, k, v, dt, a = _rand(rng, T, 1, 1, 1, P, N)
    S = np.zeros((1, 1, P, N))
    St, _ = _states(eager_fn, S, q, k, v, dt, a)
    Sh = forms.history_form(v[:, 0, 0], k[:, 0, 0], dt[:, 0, 0], a[:, 0, 0])
    _close(St[:, 0, 0], Sh)


def check_checkpoint_splits(eager_fn, seed=2):
    """Non-zero checkpoint at every split point: eager states and outputs
    equal the checkpoint+buffer route and the output-only route."""
    rng = np.random.default_rng(seed)
    T, P, N = 6, 4, 3
    q, k, v, dt, a = _rand(rng, T, 1, 1, 1, P, N)
    S_init = rng.standard_normal((1, 1, P, N))
    S = S_init.copy()
    St, yt = _states(eager_fn, S, q, k, v, dt, a)
    for split in range(T):
        S0 = S_init[0, 0] if split == 0 else St[split - 1, 0, 0]
        sl = slice(split, T)
        Sc = forms.checkpoint_form(S0, v[sl, 0, 0], k[sl, 0, 0], dt[sl, 0, 0], a[sl, 0, 0])
        _close(St[sl, 0, 0], Sc)
        yo = forms.output_only_form(S0, q[sl, 0, 0], v[sl, 0, 0], k[sl, 0, 0], dt[sl, 0, 0], a[sl, 0, 0])
        _close(yt[sl, 0, 0], yo)


def check_output_is_state_times_query(eager_fn, seed=3):
    rng = np.random.default_rng(seed)
    T, B, H, G, P, N = 5, 2, 4, 2, 3, 6
    q, k, v, dt, a = _rand(rng, T, B, H, G, P, N)
    S = rng.standard_normal((B, H, P, N))
    St, yt = _states(eager_fn, S, q, k, v, dt, a)
    for h in range(H):
        g = h * G // H
        ref = np.einsum("tbpn,tbn->tbp", St[:, :, h], q[:, :, g])
        _close(yt[:, :, h], ref)


def check_causal_linear_attention(eager_fn, seed=4):
    """a = 1, dt = 1, zero state: y_t = sum_{i<=t} v_i (k_i . q_t), i.e.
    causal (unnormalised) linear attention, Y = tril(Q K^T) V."""
    rng = np.random.default_rng(seed)
    T, P, N = 9, 4, 5
    q, k, v, _, _ = _rand(rng, T, 1, 1, 1, P, N)
    ones = np.ones((T, 1, 1))
    y = eager_fn(np.zeros((1, 1, P, N)), q, k, v, ones, ones)
    Q, K, V = q[:, 0, 0], k[:, 0, 0], v[:, 0, 0]
    ref = np.tril(Q @ K.T) @ V
    _close(y[:, 0, 0], ref)


def check_zero_decay(eager_fn, seed=5):
    """a = 0 forgets everything: y_t = dt_t v_t (k_t . q_t)."""
    rng = np.random.default_rng(seed)
    T, P, N = 6, 3, 4
    q, k, v, dt, _ = _rand(rng, T, 1, 1, 1, P, N)
    a = np.zeros((T, 1, 1))
    y = eager_fn(rng.standard_normal((1, 1, P, N)), q, k, v, dt, a)
    ref = dt[:, 0, 0, None] * v[:, 0, 0] * np.sum(k[:, 0, 0] * q[:, 0, 0], axis=1)[:, None]
    _close(y[:, 0, 0], ref)


def check_masked_matrix_form(eager_fn, seed=6):
    """General decays, zero state: Y = (M o Q K^T) (diag(dt) V) with
    M[t, i] = exp(sum_{i<j<=t} log a_j) for i <= t, from cumulative sums of
    logarithms -- a route that shares no step with the token loop."""
    rng = np.random.default_rng(seed)
    T, P, N = 10, 5, 3
    q, k, v, dt, a = _rand(rng, T, 1, 1, 1, P, N)
    y = eager_fn(np.zeros((1, 1, P, N)), q, k, v, dt, a)
    la = np.cumsum(np.log(a[:, 0, 0]))
    M = np.tril(np.exp(la[:, None] - la[None, :]))
    Q, K, V = q[:, 0, 0], k[:, 0, 0], v[:, 0, 0]
    ref = (M * (Q @ K.T)) @ (dt[:, 0, 0, None] * V)
    _close(y[:, 0, 0], ref, tol=1e-11)


def check_geometric_decay(eager_fn, seed=7):
    """Constant a from a non-zero state: y_t = a^t (S0 q_t) + sum_i a^(t-i) dt_i v_i (k_i . q_t)."""
    rng = np.random.default_rng(seed)
    T, P, N = 7, 2, 3
    aval = 0.75
    q, k, v, dt, a = _rand(rng, T, 1, 1, 1, P, N, decay=aval)
    S0 = rng.standard_normal((P, N))
    y = eager_fn(S0[None, None].copy(), q, k, v, dt, a)
    for t in range(T):
        ref = aval ** (t + 1) * (S0 @ q[t, 0, 0])
        for i in range(t + 1):
            ref = ref + aval ** (t - i) * dt[i, 0, 0] * v[i, 0, 0] * (k[i, 0, 0] @ q[t, 0, 0])
        _close(y[t, 0, 0], ref)


def check_group_sharing(eager_fn, seed=8):
    """Heads h use the k, q of group floor(h*G/H): equal to running every
    head on its own with that group's k, q (G = 1 per call)."""
    rng = np.random.default_rng(seed)
    T, B, H, G, P, N = 4, 2, 6, 3, 3, 4
    q, k, v, dt, a = _rand(rng, T, B, H, G, P, N)
    S = rng.standard_normal((B, H, P, N))
    y = eager_fn(S.copy(), q, k, v, dt, a)
    for h in range(H):
        g = (h * G) // H
        assert g == h // (H // G)
        yh = eager_fn(np.ascontiguousarray(S[:, h:h + 1]), q[:, :, g:g + 1], k[:, :, g:g + 1],
                      v[:, :, h:h + 1], dt[:, :, h:h + 1], a[:, :, h:h + 1])
        _close(y[:, :, h], yh[:, :, 0])


def check_linearity(eager_fn, seed=9):
    """y is linear in (S0, v) jointly: y(2 S0, 2 v) = 2 y(S0, v), and the
    checkpoint's contribution superposes: y(S0, v) = y(S0, 0) + y(0, v)."""
    rng = np.random.default_rng(seed)
    T, P, N = 5, 3, 4
    q, k, v, dt, a = _rand(rng, T, 1, 1, 1, P, N)
    S0 = rng.standard_normal((1, 1, P, N))
    y = eager_fn(S0.copy(), q, k, v, dt, a)
    y2 = eager_fn(2 * S0, q, k, 2 * v, dt, a)
    _close(y2, 2 * y)
    ys = eager_fn(S0.copy(), q, k, np.zeros_like(v), dt, a)
    yv = eager_fn(np.zeros_like(S0), q, k, v, dt, a)
    _close(ys + yv, y)


def load_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "worked_example_p2n2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.split() for p in line.split("|")]
            rows.append([list(map(float, p)) for p in parts])
    return rows


def check_worked_example(eager_fn):
    rows = load_worked_example()
    T = len(rows)
    a = np.array([r[0][0] for r in rows]).reshape(T, 1, 1)
    dt = np.array([r[0][1] for r in rows]).reshape(T, 1, 1)
    v = np.array([r[0][2:4] for r in rows]).reshape(T, 1, 1, 2)
    k = np.array([r[0][4:6] for r in rows]).reshape(T, 1, 1, 2)
    q = np.array([r[0][6:8] for r in rows]).reshape(T, 1, 1, 2)
    S = np.zeros((1, 1, 2, 2))
    St, yt = _states(eager_fn, S, q, k, v, dt, a)
    for t, r in enumerate(rows):
        assert np.array_equal(yt[t, 0, 0], np.array(r[1])), (t, yt[t, 0, 0], r[1])
        assert np.array_equal(St[t, 0, 0].reshape(-1), np.array(r[2])), (t, St[t, 0, 0], r[2])


ALL_CHECKS = [check_history_form, check_checkpoint_splits, check_output_is_state_times_query,
              check_causal_linear_attention, check_zero_decay, check_masked_matrix_form,
              check_geometric_decay, check_group_sharing, check_linearity, check_worked_example]
