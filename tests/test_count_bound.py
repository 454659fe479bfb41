"""Host logic: the handle's bounds on the ring counts (csrc/count_bound.h).

The bounds decide whether a flush is launched at all, so they must hold for
every sequence after every call, whatever the device does: random schedules
(appends, flushes, rollbacks, fused steps and verify rounds, with ring and
pointer overflows) run through the integer ring model of the oracle, with
the fused calls' per-sequence rules (left unchanged when they do not fit),
and after each call lo <= count <= hi and pos <= the pos bound for every
sequence; a flush with a due sequence is never skipped.  In the standard
schedule (one token per step, flush when the ring is full) the range stays
exact, so every flush but the folding one is skipped.  CPU only: the header
is compiled with g++ into a small shim."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle import ring as oring

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "linear_attention_decode_amd", "csrc")

SHIM = r"""
#include "count_bound.h"
using replay::CountBound;
extern "C" {
void *cb_new(int L) { auto *b = new CountBound; b->reset(L); return b; }
void cb_free(void *h) { delete static_cast<CountBound *>(h); }
void cb_set_pos(void *h, long long p) { static_cast<CountBound *>(h)->pos = p; }
void cb_append(void *h, int W) { static_cast<CountBound *>(h)->append(W); }
int cb_may_fold(void *h, int m) { return static_cast<CountBound *>(h)->flush_may_fold(m); }
void cb_flush(void *h, int m) { static_cast<CountBound *>(h)->flush(m); }
void cb_step(void *h, int f) { static_cast<CountBound *>(h)->step(f); }
void cb_verify_round(void *h, int f, int W) { static_cast<CountBound *>(h)->verify_round(f, W); }
void cb_rollback(void *h) { static_cast<CountBound *>(h)->rollback(); }
void cb_load(void *h) { static_cast<CountBound *>(h)->load(); }
int cb_from_pointers(void *h, const int *pos, const int *base, int B) {
    return static_cast<CountBound *>(h)->from_pointers(pos, base, B);
}
void cb_get(void *h, long long *out) {
    auto *b = static_cast<CountBound *>(h);
    out[0] = b->lo; out[1] = b->hi; out[2] = b->pos;
}
}
"""


@pytest.fixture(scope="module")
def cb(tmp_path_factory):
    d = tmp_path_factory.mktemp("cb")
    src, lib = d / "shim.cpp", d / "libcb.so"
    src.write_text(SHIM)
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(lib)],
                   check=True)
    L = ctypes.CDLL(str(lib))
    L.cb_new.restype = ctypes.c_void_p
    L.cb_from_pointers.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    for name in ("cb_free", "cb_set_pos", "cb_append", "cb_may_fold", "cb_flush", "cb_step", "cb_verify_round",
                 "cb_rollback", "cb_load", "cb_get"):
        getattr(L, name).argtypes = [ctypes.c_void_p] + {
            "cb_set_pos": [ctypes.c_longlong], "cb_append": [ctypes.c_int], "cb_may_fold": [ctypes.c_int],
            "cb_flush": [ctypes.c_int], "cb_step": [ctypes.c_int], "cb_verify_round": [ctypes.c_int, ctypes.c_int],
            "cb_get": [ctypes.POINTER(ctypes.c_longlong)]}.get(name, [])
    return L


def _get(cb, h):
    out = (ctypes.c_longlong * 3)()
    cb.cb_get(h, out)
    return int(out[0]), int(out[1]), int(out[2])


def _need(t):
    return max(int(t), 1)


def model_step(m: oring.RingModel, f: int):
    """Fused step: append one token, fold where the ring then holds >= max(f, 1)."""
    ok = ~((m.count + 1 > m.L) | (m.pos == oring.INT32_MAX))
    m.pos[ok] += 1
    fold = ok & (m.count >= _need(f))
    m.base[fold] = m.pos[fold]


def model_verify_round(m: oring.RingModel, f: int, W: int):
    """Fused verify round: fold where count >= max(f, 1), then append W; left
    unchanged when the drafts do not fit or the pointer would pass 2^31-1."""
    fold = m.count >= _need(f)
    keep = np.where(fold, 0, m.count)
    ok = ~((keep + W > m.L) | (m.pos + W > oring.INT32_MAX))
    m.base[ok & fold] = m.pos[ok & fold]
    m.pos[ok] += W


def _check(cb, h, m, what):
    lo, hi, pb = _get(cb, h)
    c = m.count
    assert 0 <= lo <= hi <= m.L, (what, lo, hi)
    assert lo <= c.min() and c.max() <= hi, (what, lo, hi, c)
    assert m.pos.max() <= pb, (what, pb, m.pos)


@pytest.mark.parametrize("L,seed,pos0", [(1, 1, 0), (4, 2, 0), (16, 3, 0), (16, 4, oring.INT32_MAX - 40),
                                         (32, 5, 0), (5, 6, oring.INT32_MAX - 7)])
def test_bounds_hold_on_random_schedules(cb, L, seed, pos0):
    rng = np.random.default_rng(seed)
    B = 6
    m = oring.RingModel(B, L, pos=[pos0] * B)
    h = cb.cb_new(L)
    cb.cb_set_pos(h, pos0)
    try:
        for it in range(3000):
            op = rng.integers(0, 7)
            if op == 0:
                W = int(rng.integers(1, L + 1))
                m.append(W)
                cb.cb_append(h, W)
            elif op == 1:
                mc = int(rng.integers(-1, L + 3))
                due = (m.count >= _need(mc)).any()
                may = cb.cb_may_fold(h, mc)
                assert may or not due, ("skipped a due flush", mc, m.count)
                m.flush(mc)
                if may:
                    cb.cb_flush(h, mc)
            elif op == 2:
                r = rng.integers(0, m.count + 2)            # sometimes past the count: rejected
                m.rollback(r)
                cb.cb_rollback(h)
            elif op == 3:
                f = int(rng.integers(-1, L + 3))
                model_step(m, f)
                cb.cb_step(h, f)
            elif op == 4:
                f = int(rng.integers(-1, L + 3))
                W = int(rng.integers(1, L + 1))
                model_verify_round(m, f, W)
                cb.cb_verify_round(h, f, W)
            elif op == 5 and rng.random() < 0.1:
                m.base[:] = m.pos                          # checkpoint load
                cb.cb_load(h)
            else:
                # the standard schedule for a while: one token a step, flush when full
                for _ in range(int(rng.integers(1, 2 * L + 2))):
                    model_step(m, L)
                    cb.cb_step(h, L)
                    _check(cb, h, m, ("standard", it))
            _check(cb, h, m, (op, it))
            m.take_error()
    finally:
        cb.cb_free(h)


@pytest.mark.parametrize("L", [1, 4, 16, 32])
def test_standard_schedule_is_exact(cb, L):
    """append(1); flush(L) per step (the copy-mode step) and the fused step:
    the range stays a single value, so only the folding flush is launched."""
    B, T = 3, 5 * L + 3
    for fused in (False, True):
        m = oring.RingModel(B, L)
        h = cb.cb_new(L)
        try:
            launched = []
            for t in range(T):
                if fused:
                    model_step(m, L)
                    cb.cb_step(h, L)
                else:
                    m.append(1)
                    cb.cb_append(h, 1)
                    may = bool(cb.cb_may_fold(h, L))
                    launched.append(may)
                    due = m.flush(L)
                    assert may == bool(due.any())
                    if may:
                        cb.cb_flush(h, L)
                lo, hi, _ = _get(cb, h)
                assert lo == hi == int(m.count[0]), (t, lo, hi, m.count)
            if not fused:
                assert sum(launched) == T // L
        finally:
            cb.cb_free(h)


def _from_pointers(cb, h, pos, base):
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    base = np.ascontiguousarray(base, dtype=np.int32)
    return bool(cb.cb_from_pointers(h, pos.ctypes.data, base.ctypes.data, len(pos)))


@pytest.mark.parametrize("L,seed", [(4, 11), (16, 12), (32, 13)])
def test_bounds_rebuilt_from_pointers(cb, L, seed):
    """replay_set_flush_skipping(1) rebuilds the range from the pointers read
    back from the device: after pointers moved behind the handle's back (a
    rollback of unknown size, an engine's own appends) the rebuilt range is
    exact -- lo and hi are the smallest and largest count -- and further
    calls keep it valid.  Pointers outside 0 <= base <= pos, count <= L are
    refused and leave the range unchanged."""
    rng = np.random.default_rng(seed)
    B = 7
    m = oring.RingModel(B, L)
    h = cb.cb_new(L)
    try:
        for it in range(400):
            # moves the handle never sees
            m.pos[:] = m.base + rng.integers(0, L + 1, size=B)
            assert _from_pointers(cb, h, m.pos, m.base)
            lo, hi, pb = _get(cb, h)
            assert (lo, hi, pb) == (int(m.count.min()), int(m.count.max()), int(m.pos.max())), it
            f = int(rng.integers(-1, L + 3))
            model_step(m, f)
            cb.cb_step(h, f)
            _check(cb, h, m, ("after rebuild", it))
            m.take_error()
        before = _get(cb, h)
        bad = [(m.pos, m.pos + 1), (m.base + L + 1, m.base), (m.pos, np.full(B, -1))]
        for pos, base in bad:
            assert not _from_pointers(cb, h, pos, base)
            assert _get(cb, h) == before
    finally:
        cb.cb_free(h)
