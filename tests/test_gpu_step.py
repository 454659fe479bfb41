"""The fused standard decode step (replay_step) on the GPU: one launch per
step that appends, decodes and, on full rings, folds the ring into the
checkpoint with the state-and-output route.  Checked against

* the separate calls (append, decode, flush) on the same inputs: outputs of
  non-folding steps and every checkpoint bit for bit, outputs of folding
  steps (a different but exact route) to 1e-5;
* the float64 oracle (1e-4 per head) and the integer ring model (exact);
* error paths: a step that would overflow the ring leaves the sequence
  unchanged and outputs NaN;
* with an e4m3 or FP4 read copy (bf16 io): append + decode from the copy in
  one launch, then the flush, against the calls in turn, bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ring as oring
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    return lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                           io_dtype=w.io_dtype, device=gu.DEV, **kw)


def _run_step(layer, w, dev, T, flush_at, model=None):
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=flush_at)
        if model is not None:
            model.append(1)
            model.flush(flush_at)
            gu.check_ring(layer, model, f"step {t}")
    return y


def test_step_matches_separate_calls_on_decode_workload():
    """Mamba-2-shaped layer (B=256, H=128, G=8, P=64, N=128, L=16), 48 steps."""
    w = synth.named("decode")
    T, L = 48, 16
    gu.note("fused step vs separate calls")
    dev = gu.DevInputs(w, 0, T)
    a = _layer(w)
    b = _layer(w)
    ya = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    yb = torch.empty_like(ya)
    for t in range(T):
        a.step(*dev.step(t), ya[t], flush_at=L)
        q, k, v, dt, aa = dev.step(t)
        b.append(1, q, k, v, dt, aa)
        b.decode(yb[t])
        b.flush(L)
        if t % L == L - 1:
            torch.cuda.synchronize()
            assert torch.equal(a.s_master, b.s_master), f"checkpoint differs after step {t}"
    torch.cuda.synchronize()
    assert a.get_error()[0] == 0 and b.get_error()[0] == 0
    assert torch.equal(a.pos, b.pos) and torch.equal(a.base, b.base)
    assert torch.equal(a.sync, torch.zeros_like(a.sync))
    folding = [t for t in range(T) if t % L == L - 1]
    plain = [t for t in range(T) if t % L != L - 1]
    assert torch.equal(ya[plain], yb[plain])
    e = runs.normwise_rel_err(ya[folding].cpu().numpy(), yb[folding].cpu().numpy().astype(np.float64))
    assert float(np.max(e)) <= 1e-5
    seqs = [0, 131, 255]
    x = gu.oracle_inputs(w, 0, T, seqs)
    y_ref = runs.standard(x, np.zeros((3, w.heads, w.head_dim, w.state_dim)))
    gu.assert_f32(ya.cpu().numpy()[:, seqs], y_ref, gu.y_abs_standard(x, (3, w.heads, w.head_dim, w.state_dim)))
    a.close()
    b.close()


@pytest.mark.parametrize("P,N,io,L,flush_at,B,H,G,copy", [
    (16, 16, "f32", 4, 4, 3, 6, 3, None),
    (64, 64, "bf16", 5, 5, 5, 4, 2, None),
    (64, 128, "f32", 7, 3, 2, 8, 4, None),
    (64, 128, "bf16", 32, 32, 2, 16, 8, None),
    (128, 128, "bf16", 8, 8, 3, 4, 2, None),
    (64, 128, "bf16", 6, 1, 3, 8, 8, None),
    (64, 128, "bf16", 8, 8, 3, 8, 2, "bf16"),
    (64, 128, "bf16", 8, 8, 3, 8, 2, "fp8"),
])
def test_step_ragged(P, N, io, L, flush_at, B, H, G, copy):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=200 + P + L + flush_at)
    T = 3 * L + 2
    gu.note(f"step {w} flush_at={flush_at} copy={copy}")
    dev = gu.DevInputs(w, 0, T)
    layer = _layer(w, read_copy=copy)
    model = oring.RingModel(B, L)
    y = _run_step(layer, w, dev, T, flush_at, model)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, T, list(range(B)))
    S0 = np.zeros((B, H, P, N))
    if copy is None:
        y_ref, tol = runs.standard(x, S0), 1e-4
    else:
        # with copies the step runs the separate kernels; with this few heads the
        # per-token error against exact is the format's own, so compare with the
        # oracle's emulation of the same copy
        y_ref, tol = runs.separated(x, S0, flush_at, copy), None
    if copy is None:
        gu.assert_f32(y.cpu().numpy(), y_ref, gu.y_abs_standard(x, (B, H, P, N)))
    else:
        gu.assert_copy(y.cpu().numpy(), y_ref, copy)
    layer.close()


def test_step_overflow_leaves_sequence_unchanged():
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=211)
    gu.note("step overflow")
    dev = gu.DevInputs(w, 0, 8)
    layer = _layer(w)
    y = torch.empty((8, 3, 4, 64), dtype=torch.float32, device=gu.DEV)
    for t in range(4):
        layer.step(*dev.step(t), y[t], flush_at=5)     # never folds: ring fills up
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    S_before = layer.s_master.clone()
    layer.step(*dev.step(4), y[4], flush_at=5)         # count would be 5 > L
    torch.cuda.synchronize()
    word, per = layer.get_error()
    assert per == [lad.SEQERR_RING_OVERFLOW] * 3
    assert torch.isnan(y[4]).all()
    assert layer.pos.cpu().tolist() == [4, 4, 4] and layer.base.cpu().tolist() == [0, 0, 0]
    assert torch.equal(layer.s_master, S_before)
    assert torch.equal(layer.sync, torch.zeros_like(layer.sync))
    # folding frees the ring and the next step proceeds
    layer.flush(1)
    layer.step(*dev.step(4), y[5], flush_at=5)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, 5, [0, 1, 2])
    y_ref = runs.standard(x, np.zeros((3, 4, 64, 128)))
    gu.assert_f32(torch.cat([y[:4], y[5:6]]).cpu().numpy(), y_ref, gu.y_abs_standard(x, (3, 4, 64, 128)))
    layer.close()


def test_flush_schedule_invariance():
    """The outputs do not depend on when the ring is folded: the same token
    stream through the fused step with flush_at = 1 (fold every step), 3 and
    L = 8 (fold when full), and through the separate calls flushing at L,
    agree with each other to float32 rounding and with the oracle (1e-4)."""
    w = synth.Workload(batch=4, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=8, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=240)
    T = 30
    gu.note("flush schedule invariance")
    dev = gu.DevInputs(w, 0, T)
    outs = {}
    for flush_at in (1, 3, 8):
        layer = _layer(w)
        outs[flush_at] = _run_step(layer, w, dev, T, flush_at).cpu().numpy()
        torch.cuda.synchronize()
        assert layer.get_error()[0] == 0
        layer.close()
    layer = _layer(w)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.append(1, *dev.step(t))
        layer.decode(y[t])
        layer.flush(w.ring_len)
    torch.cuda.synchronize()
    outs["calls"] = y.cpu().numpy()
    layer.close()
    x = gu.oracle_inputs(w, 0, T, list(range(w.batch)))
    y_ref = runs.standard(x, np.zeros((w.batch, w.heads, w.head_dim, w.state_dim)))
    y_abs = gu.y_abs_standard(x, (w.batch, w.heads, w.head_dim, w.state_dim))
    for k, yk in outs.items():
        gu.assert_f32(yk, y_ref, y_abs, what=f"schedule {k}:")
        e = runs.normwise_rel_err(yk, outs[8].astype(np.float64))
        assert float(np.max(e)) <= 1e-5, k


def test_step_ignores_nan_in_unused_slots():
    """Every ring slot starts as NaN, and after each step every slot outside
    the live range is poisoned again; the fused step's outputs and final
    checkpoint stay bit-identical to the clean run (it never reads a slot it
    must not)."""
    w = synth.Workload(batch=5, heads=8, groups=4, head_dim=64, state_dim=128, ring_len=6, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=241)
    T = 20
    gu.note("step nan poison")
    dev = gu.DevInputs(w, 0, T)

    def run(poison):
        layer = _layer(w)
        model = oring.RingModel(w.batch, w.ring_len)
        if poison:
            for name in ("ring_q", "ring_k", "ring_v", "ring_dt", "ring_a"):
                layer.t[name].fill_(float("nan"))
        y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
        for t in range(T):
            layer.step(*dev.step(t), y[t], flush_at=4)
            model.append(1)
            model.flush(4)
            if poison:
                torch.cuda.synchronize()
                for b in range(w.batch):
                    live = set(model.live_slots(b))
                    for s in range(w.ring_len):
                        if s not in live:
                            for name in ("ring_v", "ring_q", "ring_k"):
                                layer.t[name][b, :, s] = float("nan")
                            for name in ("ring_dt", "ring_a"):   # [B][L][H]
                                layer.t[name][b, s] = float("nan")
        torch.cuda.synchronize()
        assert layer.get_error()[0] == 0
        out = y.cpu().numpy(), layer.s_master.cpu().numpy()
        layer.close()
        return out

    y0, s0 = run(False)
    y1, s1 = run(True)
    assert np.isfinite(y0).all() and np.isfinite(s0).all()
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("P,N,L,flush_at,B,H,G,copy,shared", [
    (64, 128, 16, 16, 3, 16, 2, "bf16", False),    # 2 heads per workgroup
    (64, 128, 16, 16, 3, 16, 2, "fp8", False),     # 4 heads per workgroup
    (64, 128, 16, 16, 3, 16, 2, "fp4", False),
    (64, 128, 8, 5, 2, 12, 2, "fp8", False),       # 6 heads per group: one head per workgroup
    (128, 128, 32, 32, 2, 8, 2, "fp4", False),     # two ring wavefronts per head
    (16, 16, 4, 4, 3, 4, 1, "fp8", False),
    (64, 64, 12, 12, 2, 8, 2, "fp4", False),       # ring shorter than 16, 64 x 64 tiles
    (64, 64, 6, 6, 2, 8, 2, "bf16", True),         # shared: the copy is the only checkpoint
    (64, 128, 16, 16, 2, 16, 2, "fp8", True),
])
def test_copy_step_equals_calls(P, N, L, flush_at, B, H, G, copy, shared):
    """With an e4m3 or FP4 copy and bf16 io, replay_step runs append + decode
    from the copy as one launch, then the flush (a bf16 copy runs the kernels
    in turn): outputs, checkpoints, copies, scales, pointers and ring slots
    equal append, decode and flush run in turn, bit for bit."""
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=230 + P + L + flush_at)
    T = 2 * L + 3
    gu.note(f"copy step vs calls {w} flush_at={flush_at} copy={copy} shared={shared}")
    dev = gu.DevInputs(w, 0, T)
    a = _layer(w, read_copy=copy, shared_lowp=shared)
    b = _layer(w, read_copy=copy, shared_lowp=shared)
    for lay in (a, b):
        for name in ("ring_q", "ring_k", "ring_v", "ring_dt", "ring_a"):
            lay.t[name].zero_()
    ya = torch.empty((T, B, H, P), dtype=torch.float32, device=gu.DEV)
    yb = torch.empty_like(ya)
    for t in range(T):
        a.step(*dev.step(t), ya[t], flush_at=flush_at)
        b.append(1, *dev.step(t))
        b.decode(yb[t])
        b.flush(flush_at)
    torch.cuda.synchronize()
    assert a.get_error()[0] == 0 and b.get_error()[0] == 0
    assert torch.equal(ya, yb)
    assert torch.isfinite(ya).all()
    for name in ("s_master", "s_copy", "s_scale", "pos", "base", "ring_q", "ring_k", "ring_v", "ring_dt", "ring_a"):
        if a.t[name] is not None:
            assert torch.equal(a.t[name], b.t[name]), name
    assert torch.equal(a.sync, torch.zeros_like(a.sync))
    a.close()
    b.close()


def test_copy_step_overflow_gives_nan():
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=3, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=241)
    gu.note("copy step overflow")
    dev = gu.DevInputs(w, 0, 6)
    layer = _layer(w, read_copy="fp8")
    y = torch.empty((6, 3, 8, 64), dtype=torch.float32, device=gu.DEV)
    for t in range(4):
        layer.step(*dev.step(t), y[t], flush_at=5)     # never folds: ring fills up
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    ring_before = layer.ring_v.clone()
    layer.step(*dev.step(4), y[4], flush_at=5)
    torch.cuda.synchronize()
    word, per = layer.get_error()
    assert per == [lad.SEQERR_RING_OVERFLOW] * 3
    assert torch.isnan(y[4]).all() and torch.isfinite(y[:4]).all()
    assert layer.pos.cpu().tolist() == [4, 4, 4]
    assert torch.equal(layer.ring_v, ring_before)
    layer.close()
