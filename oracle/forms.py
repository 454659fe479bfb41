"""Self-check forms of the recurrence (float64, one head, small sizes) --
test infrastructure only.

These are the rewritings the pages give of the same state; the tests check
each against the eager recurrence of ``core.eager``.

* history form -- page "ReplaySSM: Cachear Inputs, No Estado", section
  "La solucion", eq. "Forma historia": from a zero initial state,
  S_t = sum_{i<=t} (prod_{i<j<=t} a_j) dt_i v_i k_i^T.
* checkpoint + buffer ("state and output") route -- same page, section
  "Los dos caminos", eq. "Ruta estado y salida": S_t = abar_t S0 +
  sum_{j=1}^{h+1} s_{j,t} v_j k_j^T, then y_t = S_t q_t.
* output-only route -- same section, eq. "Ruta solo salida":
  y_t = abar_t (S0 q) + sum_{j=1}^{h+1} s_{j,t} v_j (k_j^T q).

The extracted equations lost their subscripts ("\\bar{a}t", "\\sum{j=1}").
Reading taken: j counts the buffer entries since the checkpoint, from 1; h
entries precede the current token, which is entry t = h+1.  The pages never
define abar_t or s_{j,t}; the reading that makes the route equal the eager
recurrence started from S0 (by unrolling eq. "Forma resumen" t times) is

    abar_t  = prod_{m=1}^{t} a_m                 (includes the current a_t)
    s_{j,t} = dt_j * prod_{m=j+1}^{t} a_m        (empty product = 1)

and with S0 = 0 it reduces to eq. "Forma historia".  Products are formed
directly (no exp of sums).
"""
from __future__ import annotations

import numpy as np


def segment_decay(a: np.ndarray, dt: np.ndarray):
    """a, dt: float64 [c], buffer entries 1..c since the checkpoint.

    Returns abar [c] with abar[t-1] = prod_{m=1..t} a_m, and s [c][c] with
    s[t-1][j-1] = dt_j prod_{m=j+1..t} a_m for j <= t (zero above)."""
    c = len(a)
    abar = np.zeros(c)
    s = np.zeros((c, c))
    for t in range(1, c + 1):
        prod = 1.0
        for m in range(1, t + 1):
            prod *= a[m - 1]
        abar[t - 1] = prod
        for j in range(1, t + 1):
            w = dt[j - 1]
            for m in range(j + 1, t + 1):
                w *= a[m - 1]
            s[t - 1][j - 1] = w
    return abar, s


def history_form(v, k, dt, a):
    """Zero initial state.  v [T][P], k [T][N], dt, a [T] -> S [T][P][N]."""
    T, P = v.shape
    N = k.shape[1]
    S = np.zeros((T, P, N))
    for t in range(T):
        for i in range(t + 1):
            w = dt[i]
            for j in range(i + 1, t + 1):
                w *= a[j]
            S[t] += w * np.outer(v[i], k[i])
    return S


def checkpoint_form(S0, v, k, dt, a):
    """Buffer entries 1..c after checkpoint S0.  -> S [c][P][N] (S_t, t=1..c)."""
    c = len(a)
    abar, s = segment_decay(a, dt)
    out = np.zeros((c,) + S0.shape)
    for t in range(1, c + 1):
        St = abar[t - 1] * S0
        for j in range(1, t + 1):
            St = St + s[t - 1][j - 1] * np.outer(v[j - 1], k[j - 1])
        out[t - 1] = St
    return out


def output_only_form(S0, q, v, k, dt, a):
    """y_t for the buffer entries t=1..c, never forming S_t.  q [c][N]."""
    c = len(a)
    abar, s = segment_decay(a, dt)
    P = v.shape[1]
    y = np.zeros((c, P))
    for t in range(1, c + 1):
        qt = q[t - 1]
        yt = abar[t - 1] * (S0 @ qt)
        for j in range(1, t + 1):
            yt = yt + s[t - 1][j - 1] * v[j - 1] * float(k[j - 1] @ qt)
        y[t - 1] = yt
    return y


# ---------------------------------------------------------------------------
# Gated DeltaNet (the gated delta rule of core.eager_gdn).  The pages name the
# layer and say the replay was built for it, without its equation; these are
# the checkpoint-plus-buffer rewritings of the published rule (Yang et al.,
# ICLR 2025), derived by unrolling it -- the reading recorded for this layer:
#
#   transition  A_m = alpha_m (I - beta_m k_m k_m^T)        (N x N)
#   S_t = S0 A_1 A_2 ... A_t + sum_{j=1..t} beta_j v_j k_j^T A_{j+1} ... A_t
#
# and, applied to q_t from the right without forming S_t (the output-only
# route of this layer): with w_t = q_t and w_{m-1} = A_m w_m for m = t..1,
#
#   y_t = S0 w_0 + sum_{j=1..t} beta_j v_j (k_j . w_j)
#
# A_m w = alpha_m (w - beta_m (k_m . w) k_m) costs 2N per entry, so the chain
# is cheap next to the one pass over S0.

def gdn_transition(k, beta, alpha):
    """A = alpha (I - beta k k^T) as an explicit N x N matrix."""
    k = np.asarray(k, dtype=np.float64)
    return alpha * (np.eye(len(k)) - beta * np.outer(k, k))


def gdn_product_form(S0, v, k, beta, alpha):
    """Buffer entries 1..c after checkpoint S0, by explicit matrix products.
    v [c][P], k [c][N], beta, alpha [c] -> S [c][P][N] (S_t, t = 1..c)."""
    c = len(alpha)
    out = np.zeros((c,) + S0.shape)
    for t in range(1, c + 1):
        prod = np.eye(S0.shape[1])
        for m in range(1, t + 1):
            prod = prod @ gdn_transition(k[m - 1], beta[m - 1], alpha[m - 1])
        St = S0 @ prod
        for j in range(1, t + 1):
            tail = np.eye(S0.shape[1])
            for m in range(j + 1, t + 1):
                tail = tail @ gdn_transition(k[m - 1], beta[m - 1], alpha[m - 1])
            St = St + beta[j - 1] * np.outer(v[j - 1], k[j - 1]) @ tail
        out[t - 1] = St
    return out


def gdn_output_only_form(S0, q, v, k, beta, alpha):
    """y_t for buffer entries t = 1..c by the backward chain, never forming
    S_t or a transition matrix.  q [c][N] -> y [c][P]."""
    c = len(alpha)
    y = np.zeros((c, v.shape[1]))
    for t in range(1, c + 1):
        w = np.array(q[t - 1], dtype=np.float64)
        yt = np.zeros(v.shape[1])
        for m in range(t, 0, -1):
            d = float(k[m - 1] @ w)                   # k_m . w_m
            yt = yt + beta[m - 1] * d * v[m - 1]
            w = alpha[m - 1] * (w - beta[m - 1] * d * k[m - 1])   # w_{m-1} = A_m w_m
        y[t - 1] = yt + S0 @ w
    return y
