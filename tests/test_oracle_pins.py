"""The float64 oracle against closed forms, special cases and a hand-worked
example (no GPU).  See tests/oracle_pins.py for what each check pins."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import core
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.eager)


# --- planted mistakes ------------------------------------------------------
# Each mutant is the oracle's C source with one plausible mistake planted
# (a dropped term, a wrong sign or index, a transposed operand, a wrong
# order).  At least one pin must reject every mutant.

MUTANTS = {
    "drop_dt": ("dtt * (vt[p] * kt[n])", "(vt[p] * kt[n])"),
    "transpose_vk": ("dtt * (vt[p] * kt[n])", "dtt * (vt[n % P] * kt[p % N])"),
    "decay_of_previous_token": ("const double at = a[(t * B + b) * H + h];",
                                "const double at = a[((t > 0 ? t - 1 : 0) * B + b) * H + h];"),
    "decay_on_new_term": ("row[n] = at * row[n] + dtt * (vt[p] * kt[n]);",
                          "row[n] = at * (row[n] + dtt * (vt[p] * kt[n]));"),
    "output_before_update": ("row[n] = at * row[n] + dtt * (vt[p] * kt[n]);\n                    acc += row[n] * qt[n];",
                             "acc += row[n] * qt[n];\n                    row[n] = at * row[n] + dtt * (vt[p] * kt[n]);"),
    "sign": ("at * row[n] + dtt", "at * row[n] - dtt"),
    "no_decay": ("row[n] = at * row[n] +", "row[n] = row[n] +"),
    "group_map_modulo": ("const int64_t g = (h * G) / H;", "const int64_t g = h % G;"),
    "query_other_group": ("const double *qt = q + ((t * B + b) * G + g) * N;",
                          "const double *qt = q + ((t * B + b) * G + (G - 1 - g)) * N;"),
    "dt_of_other_head": ("const double dtt = dt[(t * B + b) * H + h];",
                         "const double dtt = dt[(t * B + b) * H + (H - 1 - h)];"),
}


def _mutant_eager(tmp_path, name):
    src = open(core._SRC).read()
    old, new = MUTANTS[name]
    # the mistake goes into oracle_eager only (other functions share lines with it)
    i = src.index("void oracle_eager(")
    j = src.index("\n}\n", i) + 3
    body = src[i:j]
    assert body.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src[:i] + body.replace(old, new) + src[j:])
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(so), str(path), "-lm"])
    L = ctypes.CDLL(str(so))
    L.oracle_eager.argtypes = [ctypes.c_int64] * 6 + [ctypes.POINTER(ctypes.c_double)] * 7
    P64 = ctypes.POINTER(ctypes.c_double)

    def eager_fn(S, q, k, v, dt, a):
        T, B, G, N = q.shape
        H, P = v.shape[2], v.shape[3]
        args = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dt, a)]
        y = np.empty((T, B, H, P))
        L.oracle_eager(T, B, H, G, P, N, *[x.ctypes.data_as(P64) for x in args],
                       S.ctypes.data_as(P64), y.ctypes.data_as(P64))
        return y
    return eager_fn


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(tmp_path, name):
    fn = _mutant_eager(tmp_path, name)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(fn)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin rejects the planted mistake {name}"


def test_oracle_threads_reported():
    assert oracle.threads() >= 1
