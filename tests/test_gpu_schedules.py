"""Random schedules through every call that moves the pointers, on the GPU.

The handle keeps host-side bounds on the ring counts and does not launch a
flush that no sequence can be due for; a flush skipped wrongly would leave
base behind.  Random calls -- fused steps (float32 checkpoint) and the
copy-mode steps (append, decode from the copy, flush), appends, rollbacks
(sometimes past the count), flushes with random thresholds, verify rounds
(fused, or the calls in turn) and decodes -- run on the device and through
the integer ring model of the oracle, with the fused calls' per-sequence
rules; pos, base and the per-sequence error bits must match after every
call.  Ring overflows happen along the way (appends past L, steps on full
rings with the fold threshold above L)."""
import numpy as np
import pytest
import torch

import synth
from oracle import ring as oring
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _need(t):
    return max(int(t), 1)


def model_step(m: oring.RingModel, f: int):
    """Fused step: append one token, fold where the ring then holds >= max(f, 1);
    a full ring (or a pointer at 2^31-1) leaves the sequence unchanged."""
    over = m.count + 1 > m.L
    big = (~over) & (m.pos == oring.INT32_MAX)
    m.err[over] |= oring.RING_OVERFLOW
    m.err[big] |= oring.POS_OVERFLOW
    ok = ~(over | big)
    m.pos[ok] += 1
    fold = ok & (m.count >= _need(f))
    m.base[fold] = m.pos[fold]


def model_verify_round(m: oring.RingModel, f: int, W: int):
    """Fused verify round: fold where count >= max(f, 1), then append W; left
    unchanged when the drafts do not fit or the pointer would pass 2^31-1."""
    fold = m.count >= _need(f)
    keep = np.where(fold, 0, m.count)
    over = keep + W > m.L
    big = (~over) & (m.pos + W > oring.INT32_MAX)
    m.err[over] |= oring.RING_OVERFLOW
    m.err[big] |= oring.POS_OVERFLOW
    ok = ~(over | big)
    m.base[ok & fold] = m.pos[ok & fold]
    m.pos[ok] += W


@pytest.mark.parametrize("io,rc,L,seed", [
    ("bf16", None, 8, 1),     # fused step, fused verify round
    ("bf16", "fp8", 8, 2),    # copy-mode step (one launch + flush), rounds as calls
    ("bf16", "bf16", 16, 3),  # bf16 copy: append, decode, flush in turn
    ("f32", None, 6, 4),      # float32 io: fused step, rounds as calls
])
def test_random_schedule_pointers(io, rc, L, seed):
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=5, heads=4, groups=2, head_dim=64, state_dim=64, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=400 + seed)
    B, H, P = w.batch, w.heads, w.head_dim
    T = 128
    gu.note(f"random schedule io={io} copy={rc} L={L}")
    dev = gu.DevInputs(w, 0, T)
    layer = lad.ReplayLayer(B, H, w.groups, P, w.state_dim, L, io_dtype=io, device=gu.DEV,
                            **({} if rc is None else {"read_copy": rc}))
    model = oring.RingModel(B, L)
    fused_step = rc is None
    fused_round = rc is None and io == "bf16" and L <= 16
    rng = np.random.default_rng(seed)
    y1 = torch.empty((B, H, P), dtype=torch.float32, device=gu.DEV)
    t = 0
    counts = {}
    for it in range(240):
        op = int(rng.choice(6, p=[0.35, 0.1, 0.15, 0.15, 0.15, 0.1]))
        counts[op] = counts.get(op, 0) + 1
        if op == 0:
            f = int(rng.integers(0, L + 3))
            layer.step(*dev.step(t), y1, flush_at=f)
            if fused_step:
                model_step(model, f)
            else:
                model.append(1)
                model.flush(f)
            t = (t + 1) % (T - 16)
        elif op == 1:
            W = int(rng.integers(1, L + 1))
            layer.append(W, *dev.window(t, W))
            model.append(W)
            t = (t + W) % (T - 16)
        elif op == 2:
            r = rng.integers(0, model.count + 2).astype(np.int32)   # sometimes past the count
            layer.rollback(torch.from_numpy(r).to(gu.DEV))
            model.rollback(r)
        elif op == 3:
            m = int(rng.integers(-1, L + 3))
            layer.flush(m)
            model.flush(m)
        elif op == 4:
            W = int(rng.integers(1, min(8, L) + 1))
            f = int(rng.integers(0, L + 3))
            yW = torch.empty((B, W, H, P), dtype=torch.float32, device=gu.DEV)
            layer.verify_step(W, *dev.window(t, W), yW, flush_at=f)
            if fused_round:
                model_verify_round(model, f, W)
            else:
                model.flush(f)
                model.append(W)
                model.read(W)
            t = (t + W) % (T - 16)
        else:
            layer.decode(y1)
            model.read(1)
        torch.cuda.synchronize()
        gu.check_ring(layer, model, f"call {it} (op {op})")
        _, per = layer.get_error()
        _, mper = model.take_error()
        assert list(per) == [int(x) for x in mper], (it, op, per, mper)
    assert all(counts.get(op, 0) > 10 for op in range(6)), counts
    layer.close()
