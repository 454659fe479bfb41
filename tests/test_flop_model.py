"""The flop half of the pages' cost model (page "ReplaySSM: Cachear Inputs,
No Estado", "Los dos caminos": the output-only route needs about 64x fewer
state-building operations at d = n = 128).  bench.py reports
flop_model(P, N); here the two routes are run as explicit loops that count
their multiply-adds on small inputs, their outputs are checked to agree
(so the loops are real evaluations of y), and the counts are checked
against the closed forms P*N and P + N per ring entry."""
import numpy as np
import pytest

import bench


class _Count:
    def __init__(self):
        self.macs = 0

    def mac(self, acc, x, y):
        self.macs += 1
        return acc + x * y


def _state_route(S0, a_bar, s, V, K, q, c):
    """y = (abar S0 + sum_j s_j v_j k_j^T) q, building the state entry by entry."""
    P, N = S0.shape
    S = a_bar * S0.copy()
    for j in range(len(s)):
        for p in range(P):
            for n in range(N):
                S[p, n] = c.mac(S[p, n], s[j] * V[j, p], K[j, n])
    return S @ q


def _output_route(S0, a_bar, s, V, K, q, c):
    """y = abar (S0 q) + sum_j s_j v_j (k_j . q), never forming the state."""
    P, N = S0.shape
    y = a_bar * (S0 @ q)
    for j in range(len(s)):
        d = 0.0
        for n in range(N):
            d = c.mac(d, K[j, n], q[n])
        for p in range(P):
            y[p] = c.mac(y[p], s[j] * d, V[j, p])
    return y


@pytest.mark.parametrize("P,N,entries", [(3, 5, 4), (8, 2, 3), (6, 6, 1)])
def test_counted_routes_match_closed_forms(P, N, entries):
    rng = np.random.default_rng(P * 100 + N)
    S0, V, K = rng.normal(size=(P, N)), rng.normal(size=(entries, P)), rng.normal(size=(entries, N))
    q, s = rng.normal(size=N), rng.uniform(0.1, 1.0, size=entries)
    cs, co = _Count(), _Count()
    ys = _state_route(S0, 0.3, s, V, K, q, cs)
    yo = _output_route(S0, 0.3, s, V, K, q, co)
    np.testing.assert_allclose(ys, yo, rtol=1e-12, atol=1e-12)
    m = bench.flop_model(P, N)
    assert cs.macs == entries * m["state_route_macs_per_entry"] == entries * P * N
    assert co.macs == entries * m["output_only_macs_per_entry"] == entries * (P + N)
    assert m["ratio"] == pytest.approx(cs.macs / co.macs, rel=1e-15)


def test_pages_figure():
    """d = n = 128 gives exactly 64, the figure the pages state."""
    assert bench.flop_model(128, 128)["ratio"] == 64.0
    assert bench.flop_model(64, 128)["ratio"] == pytest.approx(8192 / 192)
