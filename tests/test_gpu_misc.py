"""GPU tests of the remaining entry points and edge cases: the eager
baseline, full-length decode at the benchmarked size, error paths, NaN
poisoning of unused ring slots, checkpoint save / resume, the stream probe."""
import numpy as np
import pytest
import torch

import synth
from oracle import ring as oring
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _lad():
    import linear_attention_decode_amd as lad
    return lad


def _layer(w, **kw):
    return _lad().ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                              io_dtype=w.io_dtype, device=gu.DEV, **kw)


def test_decode_workload_full_length():
    """Mamba-2-shaped layer at the benchmarked size and schedule: B=256,
    H=128, G=8, P=64, N=128, L=16, 256 steps (16 flushes), the launch
    sequence bench.py times; 4 sampled sequences against the oracle, the
    ring integers of all sequences checked after every call."""
    w = synth.named("decode")
    T, seqs = 256, [0, 63, 191, 255]
    gu.note("decode full length")
    dev = synth.step_inputs_torch(w, 0, T, device=gu.DEV)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.append(1, dev["q"][t], dev["k"][t], dev["v"][t], dev["dt"][t], dev["a"][t])
        layer.decode(y[t])
        layer.flush(w.ring_len)
        model.append(1)
        model.read(1)
        model.flush(w.ring_len)
        if t % 16 == 15:
            gu.check_ring(layer, model, f"step {t}")
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = runs.widen_inputs({k: synth.to_storage(v[:, seqs]) for k, v in dev.items()}, w.io_dtype)
    S = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_ref = runs.standard(x, S)
    gu.assert_f32(y.cpu().numpy()[:, seqs], y_ref, gu.y_abs_standard(x, S.shape))
    S_gpu = layer.s_master.cpu().numpy()[seqs].astype(np.float64)
    assert float(np.max(runs.normwise_rel_err(S_gpu, S, axes=(-3, -2, -1)))) <= 1e-4
    layer.close()


@pytest.mark.parametrize("P,N,io", [(64, 128, "bf16"), (16, 16, "f32"), (128, 128, "bf16")])
def test_eager_step_and_select(P, N, io):
    """The eager baseline: in-place steps against the oracle, then a
    speculative round with snapshots restored per sequence."""
    lad = _lad()
    w = synth.Workload(batch=5, heads=8, groups=2, head_dim=P, state_dim=N, ring_len=4, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=71)
    T = 6
    gu.note(f"eager {P}x{N} {io}")
    dev = gu.DevInputs(w, 0, T)
    cfg = lad.ReplayConfig(w.batch, w.heads, w.groups, P, N, 4, lad.BF16 if io == "bf16" else lad.F32,
                           lad.NONE, 0)
    S = torch.zeros((w.batch, w.heads, P, N), dtype=torch.float32, device=gu.DEV)
    y = torch.empty((T, w.batch, w.heads, P), dtype=torch.float32, device=gu.DEV)
    for t in range(3):
        lad.replay_eager_step(cfg, S, S, *dev.step(t), y[t])
    # round of 3 drafts written to snapshots, then restore snapshot c_b - 1
    snaps = torch.empty((3,) + tuple(S.shape), dtype=torch.float32, device=gu.DEV)
    for i in range(3):
        lad.replay_eager_step(cfg, S if i == 0 else snaps[i - 1], snaps[i], *dev.step(3 + i), y[3 + i])
    accept = np.array([0, 1, 2, 3, 2], dtype=np.int32)
    lad.replay_eager_select(cfg, snaps, 3, torch.from_numpy(accept).to(gu.DEV), S)
    torch.cuda.synchronize()
    x = gu.oracle_inputs(w, 0, T, list(range(w.batch)))
    S_ref = np.zeros((w.batch, w.heads, P, N))
    y_ref = runs.standard(x, S_ref.copy())
    gu.assert_f32(y.cpu().numpy(), y_ref, gu.y_abs_standard(x, S_ref.shape))
    for b in range(w.batch):
        Sb = np.zeros((1, w.heads, P, N))
        runs.standard({k: v[:3 + accept[b], [b]] for k, v in x.items()}, Sb)
        e = runs.normwise_rel_err(S[b].cpu().numpy().astype(np.float64), Sb[0], axes=(-3, -2, -1))
        assert float(e) <= 1e-5, (b, float(e))


def test_error_paths_leave_sequences_unchanged():
    """Ring overflow, rollback out of range, too few entries for a window and
    a pointer at its limit set the documented bits for exactly the sequences
    concerned; those sequences' pointers, checkpoints and outputs of other
    sequences are unchanged."""
    lad = _lad()
    w = synth.Workload(batch=4, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=81)
    gu.note("error paths")
    dev = gu.DevInputs(w, 0, 8)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    for t in range(3):
        layer.append(1, *dev.step(t))
        model.append(1)
    # overflow: append 2 on top of 3 (L=4) fails for every sequence
    layer.append(2, *dev.window(3, 2))
    model.append(2)
    gu.check_ring(layer, model, "overflow")
    word, per = layer.get_error()
    assert word == lad.SEQERR_RING_OVERFLOW and per == [lad.SEQERR_RING_OVERFLOW] * 4
    # rollback with per-sequence counts: 4 > count(3) and -1 are rejected
    r = np.array([1, 4, -1, 3], dtype=np.int32)
    layer.rollback(torch.from_numpy(r).to(gu.DEV))
    model.rollback(r)
    gu.check_ring(layer, model, "rollback")
    word, per = layer.get_error()
    assert per == [0, lad.SEQERR_ROLLBACK_RANGE, lad.SEQERR_ROLLBACK_RANGE, 0]
    # verify a window of 3 with counts [2, 3, 3, 0]: sequences 0 and 3 fail, NaN outputs
    y = torch.zeros((4, 3, 4, 64), dtype=torch.float32, device=gu.DEV)
    layer.verify(3, y)
    torch.cuda.synchronize()
    word, per = layer.get_error()
    assert per == [lad.SEQERR_TOO_FEW, 0, 0, lad.SEQERR_TOO_FEW]
    yc = y.cpu().numpy()
    assert np.isnan(yc[[0, 3]]).all() and np.isfinite(yc[[1, 2]]).all()
    # flush on an empty ring is a no-op; a pointer at 2^31-1 cannot advance
    layer.flush(1)
    model.flush(1)
    layer.pos[3] = 2 ** 31 - 1
    layer.base[3] = 2 ** 31 - 1
    model.pos[3] = model.base[3] = 2 ** 31 - 1
    layer.append(1, *dev.step(7))
    model.append(1)
    gu.check_ring(layer, model, "pos overflow")
    word, per = layer.get_error()
    assert per == [0, 0, 0, lad.SEQERR_POS_OVERFLOW]
    assert layer.get_error()[0] == 0          # reading cleared them
    layer.close()


def test_nan_poisoned_unused_slots_change_nothing():
    """Ring slots outside the live range, and drafts rejected by a rollback,
    are overwritten with NaN; every output stays bit-identical to the
    unpoisoned run (no kernel reads a slot it must not)."""
    w = synth.Workload(batch=6, heads=8, groups=4, head_dim=64, state_dim=128, ring_len=8,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=91)
    R, W = 10, 3
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    gu.note("nan poison")

    def run(poison):
        layer = _layer(w)
        model = oring.RingModel(w.batch, w.ring_len)
        if poison:
            for name in ("ring_q", "ring_k", "ring_v", "ring_dt", "ring_a"):
                layer.t[name].fill_(float("nan"))
        ys = []
        nrej = torch.from_numpy((W - accept).astype(np.int32)).to(gu.DEV)
        for r in range(R):
            layer.flush(w.ring_len - W + 1)
            model.flush(w.ring_len - W + 1)
            layer.append(W, *dev.window(r * W, W))
            model.append(W)
            y = torch.empty((w.batch, W, w.heads, 64), dtype=torch.float32, device=gu.DEV)
            layer.verify(W, y)
            ys.append(y)
            layer.rollback(nrej[r])
            model.rollback(W - accept[r])
            if poison:
                torch.cuda.synchronize()
                for b in range(w.batch):
                    live = set(model.live_slots(b))
                    for s in range(w.ring_len):
                        if s not in live:
                            layer.t["ring_v"][b, :, s] = float("nan")
                            for name in ("ring_dt", "ring_a"):   # [B][L][H]
                                layer.t[name][b, s] = float("nan")
                    # the group rows too, when no live entry uses the slot
                    for s in range(w.ring_len):
                        if s not in live:
                            layer.t["ring_q"][b, :, s] = float("nan")
                            layer.t["ring_k"][b, :, s] = float("nan")
        layer.flush(1)
        torch.cuda.synchronize()
        out = torch.stack(ys).cpu().numpy(), layer.s_master.cpu().numpy()
        assert layer.get_error()[0] == 0
        layer.close()
        return out

    y0, s0 = run(False)
    y1, s1 = run(True)
    assert np.isfinite(y0).all() and np.isfinite(s0).all()
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)


def test_checkpoint_save_and_resume():
    """Flush, save the checkpoint, load it into a fresh layer and continue:
    outputs equal the uninterrupted run's bit for bit."""
    w = synth.Workload(batch=4, heads=16, groups=4, head_dim=64, state_dim=128, ring_len=8,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=92)
    T1, T2 = 13, 11
    dev = gu.DevInputs(w, 0, T1 + T2)
    gu.note("checkpoint resume")
    full = _layer(w)
    y_full = gu.run_standard(full, w, dev, 0, T1)
    full.flush(1)
    saved = full.s_master.clone()
    y_full2 = gu.run_standard(full, w, dev, T1, T1 + T2)
    resumed = _layer(w)
    resumed.load_checkpoint(saved)
    y_res = gu.run_standard(resumed, w, dev, T1, T1 + T2)
    torch.cuda.synchronize()
    assert np.array_equal(y_full2.cpu().numpy(), y_res.cpu().numpy())
    assert resumed.get_error()[0] == 0 and full.get_error()[0] == 0
    full.close()
    resumed.close()


def test_stream_probe_copy():
    lad = _lad()
    n = (64 << 20) + 48
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=gu.DEV)
    dst = torch.zeros_like(src)
    lad.replay_stream_probe(1, src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    out = torch.zeros((n + 32767) // 32768, dtype=torch.float32, device=gu.DEV)
    lad.replay_stream_probe(0, src, out, n)
    torch.cuda.synchronize()


def test_flush_skipping_for_pointers_moved_outside_the_library():
    """An engine that moves pos itself (here: two tokens appended behind the
    handle's back) makes the handle's count bounds stale, so a due flush
    would be skipped.  replay_set_flush_skipping(0) enqueues every flush (the
    ring folds); replay_set_flush_skipping(1) reads the pointers back and
    skips again where nothing can be due; pos and base follow the integer
    ring model throughout."""
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=93)
    gu.note("flush skipping with external pointer moves")
    dev = gu.DevInputs(w, 0, 12)
    layer = _layer(w)
    for name in ("ring_q", "ring_k", "ring_v", "ring_dt", "ring_a"):
        layer.t[name].zero_()
    model = oring.RingModel(w.batch, w.ring_len)
    for t in range(2):
        layer.append(1, *dev.step(t))
        model.append(1)
    torch.cuda.synchronize()
    layer.pos += 2                      # the engine's own appends (zeroed slots)
    model.pos += 2
    layer.set_flush_skipping(False)
    layer.flush(4)                      # due on the device; the handle's bounds say count 2
    model.flush(4)
    gu.check_ring(layer, model, "flush with skipping off")
    assert layer.base.cpu().tolist() == [4, 4, 4]
    layer.set_flush_skipping(True)      # bounds rebuilt from the device: count 0 everywhere
    for t in range(2, 6):
        layer.append(1, *dev.step(t))
        model.append(1)
        layer.flush(4)
        model.flush(4)
        gu.check_ring(layer, model, f"step {t} after the rebuild")
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    assert layer.base.cpu().tolist() == [8, 8, 8]
    assert torch.isfinite(layer.s_master).all()
    layer.close()
