"""Pins of the float64 gated-delta-rule oracle (core.eager_gdn) against
things other than itself.

The pages name Gated DeltaNet as the second layer type the replay serves
and print no equation for it; the oracle follows the published gated delta
rule (Yang, Kautz, Hatamizadeh, "Gated Delta Networks: Improving Mamba2
with Delta Rule", ICLR 2025):

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   y_t = S_t q_t

Each check takes ``eager_fn(S, q, k, v, beta, alpha) -> y`` so the same
checks run against builds of the oracle with planted mistakes
(tests/test_oracle_gdn.py).  What pins what:

* zero beta: the rule degenerates to pure decay, S_t = (prod alpha) S_0;
* alpha = beta = 1 with unit keys: the update writes v_t at key k_t exactly,
  S_t k_t = v_t (the delta rule's defining property);
* orthonormal keys, alpha = beta = 1, S_0 = 0: writes do not interfere,
  y_t = sum_{j<=t} v_j (k_j . q_t);
* alpha = 1, beta = 2, v = 0, unit keys: I - 2 k k^T is a reflection, the
  state's Frobenius norm is kept;
* a hand-worked two-token example (values below, worked by hand);
* the explicit matrix-product form and the backward-chain output-only form
  of oracle.forms (written from the unrolled rule, sharing no code with the
  C recurrence);
* group sharing: head h reads the q, k of group h*G/H.
"""
from __future__ import annotations

import numpy as np

from oracle import forms


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(rng, T, B, H, G, P, N, unit=True):
    q = rng.standard_normal((T, B, G, N))
    k = rng.standard_normal((T, B, G, N))
    if unit:
        k = _unit(k)
    v = rng.standard_normal((T, B, H, P))
    beta = rng.uniform(0.05, 0.95, (T, B, H))
    alpha = rng.uniform(0.3, 0.99, (T, B, H))
    return q, k, v, beta, alpha


def check_zero_beta_is_pure_decay(eager_fn):
    rng = np.random.default_rng(11)
    T, B, H, G, P, N = 5, 2, 2, 1, 3, 4
    q, k, v, beta, alpha = _rand(rng, T, B, H, G, P, N)
    beta[:] = 0.0
    S0 = rng.standard_normal((B, H, P, N))
    S = S0.copy()
    y = eager_fn(S, q, k, v, beta, alpha)
    cum = np.cumprod(alpha, axis=0)                          # [T][B][H]
    for t in range(T):
        for b in range(B):
            for h in range(H):
                ref = cum[t, b, h] * (S0[b, h] @ q[t, b, 0])
                assert np.allclose(y[t, b, h], ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, cum[-1][..., None, None] * S0, rtol=1e-12, atol=1e-12)


def check_writes_value_at_key(eager_fn):
    rng = np.random.default_rng(12)
    B, H, G, P, N = 1, 2, 1, 3, 5
    S = rng.standard_normal((B, H, P, N))
    for t in range(4):
        q, k, v, beta, alpha = _rand(rng, 1, B, H, G, P, N)
        beta[:] = 1.0
        alpha[:] = 1.0
        eager_fn(S, q, k, v, beta, alpha)
        for h in range(H):
            assert np.allclose(S[0, h] @ k[0, 0, 0], v[0, 0, h], rtol=1e-12, atol=1e-12)


def check_orthonormal_keys_accumulate(eager_fn):
    rng = np.random.default_rng(13)
    T, B, H, G, P, N = 4, 1, 1, 1, 3, 6
    q, k, v, beta, alpha = _rand(rng, T, B, H, G, P, N)
    k[:] = 0.0
    for t in range(T):
        k[t, 0, 0, N - 1 - t] = 1.0                          # distinct one-hot keys (T <= N)
    beta[:] = 1.0
    alpha[:] = 1.0
    S = np.zeros((B, H, P, N))
    y = eager_fn(S, q, k, v, beta, alpha)
    for t in range(T):
        ref = sum(v[j, 0, 0] * float(k[j, 0, 0] @ q[t, 0, 0]) for j in range(t + 1))
        assert np.allclose(y[t, 0, 0], ref, rtol=1e-12, atol=1e-12)


def check_reflection_keeps_norm(eager_fn):
    rng = np.random.default_rng(14)
    T, B, H, G, P, N = 6, 1, 1, 1, 4, 5
    q, k, v, beta, alpha = _rand(rng, T, B, H, G, P, N)
    beta[:] = 2.0
    alpha[:] = 1.0
    v[:] = 0.0
    S = rng.standard_normal((B, H, P, N))
    n0 = np.linalg.norm(S)
    for t in range(T):
        eager_fn(S, q[t:t + 1], k[t:t + 1], v[t:t + 1], beta[t:t + 1], alpha[t:t + 1])
        assert abs(np.linalg.norm(S) - n0) <= 1e-12 * n0


def check_hand_example(eager_fn):
    # Worked by hand.  S_0 = [[1, 0], [0, 2]].
    # Token 1: k = (1, 0), beta = 1/2, alpha = 1/2, v = (2, 4), q = (1, 1):
    #   row 0: s.k = 1 -> 1/2 ((1,0) - 1/2 (1,0)) + 1/2*2 (1,0) = (5/4, 0)
    #   row 1: s.k = 0 -> 1/2 (0, 2) + 1/2*4 (1, 0)             = (2, 1)
    #   y = (5/4, 3)
    # Token 2: k = (3/5, 4/5), beta = 1, alpha = 1, v = (0, 0), q = (4/5, -3/5):
    #   row 0: s.k = 3/4 -> (5/4, 0) - 3/4 (3/5, 4/5) = (4/5, -3/5)
    #   row 1: s.k = 2   -> (2, 1) - 2 (3/5, 4/5)     = (4/5, -3/5)
    #   y = (16/25 + 9/25, same) = (1, 1)
    S = np.array([[[[1.0, 0.0], [0.0, 2.0]]]])
    q = np.array([[[[1.0, 1.0]]], [[[0.8, -0.6]]]])
    k = np.array([[[[1.0, 0.0]]], [[[0.6, 0.8]]]])
    v = np.array([[[[2.0, 4.0]]], [[[0.0, 0.0]]]])
    beta = np.array([[[0.5]], [[1.0]]])
    alpha = np.array([[[0.5]], [[1.0]]])
    y = eager_fn(S, q, k, v, beta, alpha)
    assert np.allclose(y[0, 0, 0], [1.25, 3.0], rtol=0, atol=1e-14)
    assert np.allclose(y[1, 0, 0], [1.0, 1.0], rtol=0, atol=1e-14)
    assert np.allclose(S[0, 0], [[0.8, -0.6], [0.8, -0.6]], rtol=0, atol=1e-14)


def check_product_form(eager_fn):
    rng = np.random.default_rng(15)
    for unit in (True, False):
        T, B, H, G, P, N = 5, 1, 1, 1, 3, 4
        q, k, v, beta, alpha = _rand(rng, T, B, H, G, P, N, unit=unit)
        S0 = rng.standard_normal((P, N))
        S = S0[None, None].copy()
        states = []
        for t in range(T):
            eager_fn(S, q[t:t + 1], k[t:t + 1], v[t:t + 1], beta[t:t + 1], alpha[t:t + 1])
            states.append(S[0, 0].copy())
        ref = forms.gdn_product_form(S0, v[:, 0, 0], k[:, 0, 0], beta[:, 0, 0], alpha[:, 0, 0])
        assert np.allclose(np.stack(states), ref, rtol=1e-11, atol=1e-12)


def check_output_only_chain(eager_fn):
    rng = np.random.default_rng(16)
    T, B, H, G, P, N = 7, 1, 1, 1, 4, 6
    q, k, v, beta, alpha = _rand(rng, T, B, H, G, P, N)
    S0 = rng.standard_normal((P, N))
    y = eager_fn(S0[None, None].copy(), q, k, v, beta, alpha)
    ref = forms.gdn_output_only_form(S0, q[:, 0, 0], v[:, 0, 0], k[:, 0, 0], beta[:, 0, 0], alpha[:, 0, 0])
    assert np.allclose(y[:, 0, 0], ref, rtol=1e-11, atol=1e-12)


def check_group_sharing(eager_fn):
    rng = np.random.default_rng(17)
    T, B, H, G, P, N = 3, 2, 6, 3, 2, 3
    q, k, v, beta, alpha = _rand(rng, T, B, H, G, P, N)
    S0 = rng.standard_normal((B, H, P, N))
    y = eager_fn(S0.copy(), q, k, v, beta, alpha)
    for h in range(H):
        g = (h * G) // H
        for b in range(B):
            ref = forms.gdn_output_only_form(S0[b, h], q[:, b, g], v[:, b, h], k[:, b, g], beta[:, b, h],
                                             alpha[:, b, h])
            assert np.allclose(y[:, b, h], ref, rtol=1e-11, atol=1e-12)


ALL_CHECKS = [check_zero_beta_is_pure_decay, check_writes_value_at_key, check_orthonormal_keys_accumulate,
              check_reflection_keeps_norm, check_hand_example, check_product_form, check_output_only_chain,
              check_group_sharing]
