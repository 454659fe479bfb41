"""Integer model of the input ring and its pointer -- test infrastructure.

The pages describe the state as a checkpoint plus a buffer of the most recent
inputs with a pointer: decoding appends to the buffer and flushes it into the
checkpoint when it is full (page "ReplaySSM: Cachear Inputs, No Estado",
section "Como funciona en la practica", "Decodificacion estandar"); a
rejected speculative token is undone by moving the buffer pointer back
(same section, "Rollback"; page "The SSM Layer Nobody Made Fast (Until Now):
ReplaySSM Explained", key technical takeaways: an O(1) pointer decrement).
The ring length L (e.g. 16) is from the same takeaways list.

Reading taken (the pages give no pointer arithmetic):
  pos   tokens appended and not rolled back since the start, per sequence
  base  pos at the last flush; count = pos - base entries are buffered
  token with absolute index n lives in ring slot n mod L
  append(W)   needs count + W <= L (else RING_OVERFLOW) and pos + W < 2^31
              (else POS_OVERFLOW); then pos += W
  rollback(r) needs 0 <= r <= count (else ROLLBACK_RANGE); then pos -= r
  flush(m)    if count >= max(m, 1): base = pos; otherwise nothing
  decode / verify(W) need count >= W (else TOO_FEW)
A call that fails for a sequence sets that sequence's error bit and leaves
it unchanged.  Parity pinned by hand-worked schedules and invariants in
tests/test_ring_model.py.
"""
from __future__ import annotations

import numpy as np

RING_OVERFLOW = 1
ROLLBACK_RANGE = 2
TOO_FEW = 4
POS_OVERFLOW = 8
INT32_MAX = 2 ** 31 - 1


class RingModel:
    def __init__(self, batch: int, ring_len: int, pos=None):
        self.L = int(ring_len)
        self.pos = np.zeros(batch, dtype=np.int64) if pos is None else np.array(pos, dtype=np.int64)
        self.base = self.pos.copy()
        self.err = np.zeros(batch, dtype=np.int64)

    @property
    def count(self) -> np.ndarray:
        return self.pos - self.base

    def append(self, W: int) -> np.ndarray:
        over = self.count + W > self.L
        big = (~over) & (self.pos + W > INT32_MAX)
        ok = ~(over | big)
        self.err[over] |= RING_OVERFLOW
        self.err[big] |= POS_OVERFLOW
        slots = [(self.pos + i) % self.L for i in range(W)]
        self.pos[ok] += W
        return ok, slots

    def rollback(self, r) -> np.ndarray:
        r = np.broadcast_to(np.asarray(r, dtype=np.int64), self.pos.shape)
        bad = (r < 0) | (r > self.count)
        self.err[bad] |= ROLLBACK_RANGE
        self.pos[~bad] -= r[~bad]
        return ~bad

    def flush(self, min_count: int) -> np.ndarray:
        due = self.count >= max(int(min_count), 1)
        self.base[due] = self.pos[due]
        return due

    def read(self, W: int) -> np.ndarray:
        few = self.count < W
        self.err[few] |= TOO_FEW
        return ~few

    def live_slots(self, b: int):
        """Ring slots holding entries 1..count of sequence b, oldest first."""
        return [int((self.base[b] + j) % self.L) for j in range(int(self.count[b]))]

    def take_error(self) -> int:
        word = int(np.bitwise_or.reduce(self.err)) if self.err.size else 0
        per = self.err.copy()
        self.err[:] = 0
        return word, per
