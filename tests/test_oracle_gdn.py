"""The float64 gated-delta-rule oracle against closed forms, invariants, a
hand-worked example and independent forms (no GPU); planted mistakes in
copies of its C source must each fail at least one pin.  See
tests/oracle_gdn_pins.py for what each check pins."""
import ctypes
import subprocess

import numpy as np
import pytest

import oracle
from oracle import core
from tests import oracle_gdn_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_gdn_oracle_pin(check):
    check(oracle.eager_gdn)


# Each mutant plants one plausible mistake in oracle_eager_gdn (a dropped
# factor, a wrong sign, operand or index, a wrong order).
MUTANTS = {
    "dot_with_query": ("for (int64_t n = 0; n < N; ++n) sk += row[n] * kt[n];",
                       "for (int64_t n = 0; n < N; ++n) sk += row[n] * qt[n];"),
    "no_alpha_on_correction": ("row[n] = al * (row[n] - be * sk * kt[n]) + be * vt[p] * kt[n];",
                               "row[n] = al * row[n] - be * sk * kt[n] + be * vt[p] * kt[n];"),
    "alpha_on_write": ("row[n] = al * (row[n] - be * sk * kt[n]) + be * vt[p] * kt[n];",
                       "row[n] = al * (row[n] - be * sk * kt[n] + be * vt[p] * kt[n]);"),
    "no_beta_on_write": ("+ be * vt[p] * kt[n];", "+ vt[p] * kt[n];"),
    "no_beta_on_correction": ("row[n] - be * sk * kt[n]", "row[n] - sk * kt[n]"),
    "sign": ("row[n] - be * sk * kt[n]", "row[n] + be * sk * kt[n]"),
    "transpose_write": ("+ be * vt[p] * kt[n];", "+ be * vt[n % P] * kt[p % N];"),
    "beta_alpha_swapped": ("const double al = alpha[(t * B + b) * H + h];",
                           "const double al = beta[(t * B + b) * H + h];"),
    "output_before_update": ("row[n] = al * (row[n] - be * sk * kt[n]) + be * vt[p] * kt[n];\n"
                             "                    acc += row[n] * qt[n];",
                             "acc += row[n] * qt[n];\n"
                             "                    row[n] = al * (row[n] - be * sk * kt[n]) + be * vt[p] * kt[n];"),
    "group_map_modulo": None,   # filled below: the gdn function's own group line
}


def _gdn_source():
    src = open(core._SRC).read()
    i = src.index("void oracle_eager_gdn(")
    j = src.index("\n}\n", i) + 3
    return src, i, j


def _mutant(tmp_path, name):
    src, i, j = _gdn_source()
    body = src[i:j]
    if name == "group_map_modulo":
        old, new = "const int64_t g = (h * G) / H;", "const int64_t g = h % G;"
    else:
        old, new = MUTANTS[name]
    assert body.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src[:i] + body.replace(old, new) + src[j:])
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(so), str(path), "-lm"])
    L = ctypes.CDLL(str(so))
    P64 = ctypes.POINTER(ctypes.c_double)
    L.oracle_eager_gdn.argtypes = [ctypes.c_int64] * 6 + [P64] * 7

    def eager_fn(S, q, k, v, beta, alpha):
        T, B, G, N = q.shape
        H, P = v.shape[2], v.shape[3]
        args = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, beta, alpha)]
        y = np.empty((T, B, H, P))
        L.oracle_eager_gdn(T, B, H, G, P, N, *[x.ctypes.data_as(P64) for x in args],
                           S.ctypes.data_as(P64), y.ctypes.data_as(P64))
        return y
    return eager_fn


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gdn_pins_reject_planted_mistake(tmp_path, name):
    fn = _mutant(tmp_path, name)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(fn)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin rejects the planted mistake {name}"


def test_gdn_zero_key_row_is_pure_decay_of_the_other_rows():
    """k = 0 leaves only the decay: the same as beta = 0 (no write, no erase)."""
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((1, 2, 3, 4))
    q = rng.standard_normal((2, 1, 1, 4))
    k = np.zeros((2, 1, 1, 4))
    v = rng.standard_normal((2, 1, 2, 3))
    beta = np.full((2, 1, 2), 0.7)
    alpha = np.full((2, 1, 2), 0.5)
    S = S0.copy()
    oracle.eager_gdn(S, q, k, v, beta, alpha)
    assert np.allclose(S, 0.25 * S0, rtol=0, atol=1e-15)
