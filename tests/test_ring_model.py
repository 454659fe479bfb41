"""The integer ring/pointer model against hand-worked schedules and its
invariants (no GPU)."""
import numpy as np

from oracle.ring import (POS_OVERFLOW, RING_OVERFLOW, ROLLBACK_RANGE, TOO_FEW, INT32_MAX,
                         RingModel)


def test_hand_worked_standard_schedule():
    # L = 4: append one token, read it, flush when the ring is full
    m = RingModel(1, 4)
    trace = []
    for _ in range(9):
        m.append(1)
        m.read(1)
        m.flush(4)
        trace.append((int(m.pos[0]), int(m.base[0])))
    assert trace == [(1, 0), (2, 0), (3, 0), (4, 4), (5, 4), (6, 4), (7, 4), (8, 8), (9, 8)]
    assert m.take_error()[0] == 0


def test_hand_worked_speculative_schedule():
    # L = 8, W = 3: flush(L-W+1) before appending, then reject some drafts
    m = RingModel(2, 8)
    accept = [[3, 0], [1, 2], [3, 3], [0, 1]]
    trace = []
    for c in accept:
        m.flush(8 - 3 + 1)
        ok, slots = m.append(3)
        assert ok.all()
        m.read(3)
        m.rollback(3 - np.array(c))
        trace.append((m.pos.tolist(), m.base.tolist()))
    assert trace == [([3, 0], [0, 0]),
                     ([4, 2], [0, 0]),
                     ([7, 5], [0, 0]),
                     ([7, 6], [7, 0])]
    # sequence 0 flushed at pos 7 (count 7 >= 6) before the 4th round, then
    # appended 3 and rejected all 3
    assert m.take_error()[0] == 0


def test_slots_wrap_modulo_L():
    m = RingModel(1, 4, pos=[6])
    ok, slots = m.append(3)
    assert [int(s[0]) for s in slots] == [2, 3, 0]
    assert m.live_slots(0) == [2, 3, 0]


def test_overflow_and_range_errors_leave_sequence_unchanged():
    m = RingModel(3, 4)
    m.append(3)
    ok, _ = m.append(2)                    # 3 + 2 > 4
    assert not ok.any()
    assert m.pos.tolist() == [3, 3, 3]
    m.rollback([4, 3, -1])                 # 4 > count, -1 < 0
    assert m.pos.tolist() == [3, 0, 3]
    m.read(1)
    word, per = m.take_error()
    assert per.tolist() == [RING_OVERFLOW | ROLLBACK_RANGE, RING_OVERFLOW | TOO_FEW,
                            RING_OVERFLOW | ROLLBACK_RANGE]
    assert word == RING_OVERFLOW | ROLLBACK_RANGE | TOO_FEW
    assert m.take_error()[0] == 0          # reading clears


def test_flush_on_empty_ring_is_noop_and_min_count():
    m = RingModel(2, 8)
    m.flush(0)
    assert m.base.tolist() == [0, 0]
    m.append(2)
    m.rollback([0, 2])
    m.flush(2)
    assert m.base.tolist() == [2, 0] and m.pos.tolist() == [2, 0]


def test_pos_overflow():
    m = RingModel(1, 16, pos=[INT32_MAX - 1])
    ok, _ = m.append(1)
    assert ok.all()
    ok, _ = m.append(1)
    assert not ok.any()
    assert m.take_error()[1].tolist() == [POS_OVERFLOW]


def test_random_schedules_keep_invariants():
    rng = np.random.default_rng(5)
    for trial in range(20):
        B, L = 7, int(rng.integers(1, 12))
        m = RingModel(B, L)
        for _ in range(200):
            op = rng.integers(0, 3)
            before = (m.pos.copy(), m.base.copy())
            if op == 0:
                W = int(rng.integers(1, L + 1))
                ok, _ = m.append(W)
                assert np.all(m.pos[ok] == before[0][ok] + W)
                assert np.all(m.pos[~ok] == before[0][~ok])
            elif op == 1:
                r = rng.integers(-1, L + 2, size=B)
                ok = m.rollback(r)
                assert np.all(m.pos[ok] == before[0][ok] - r[ok])
                assert np.all(m.pos[~ok] == before[0][~ok])
            else:
                mc = int(rng.integers(0, L + 1))
                due = m.flush(mc)
                assert np.all(m.base[due] == m.pos[due])
                assert np.all(m.base[~due] == before[1][~due])
            c = m.count
            assert np.all((c >= 0) & (c <= L))
            assert np.all(m.base >= 0)
