"""Every sequence of the full batch against the float64 oracle.

The other workload-size tests sample a few sequences; per-sequence index
arithmetic (the XCD-aware workgroup order, the writer workgroups that
follow the compute grid, the per-sequence arrival counters, pointer reads)
is covered here on all of them:

* standard decode (B=256, H=128, G=8, P=64, N=128, L=16, bf16 q/k/v,
  float32 checkpoint), 64 steps (4 folds) through the fused replay_step, the
  launch sequence the benchmark times: every output of every sequence and
  head within 1e-4 per head (max_p |y - y_ref| / max_p |y_ref|, floored at
  1 % of the head's term magnitude: tests/parity.py), and every checkpoint
  after the last fold within 1e-4 of the oracle state;
* the same decode layer reading an e4m3 or MX-FP4 copy of its float32
  checkpoint (separated precisions: the copy-mode step, then the flush), 32
  steps (2 folds): every output of every sequence against the oracle's
  emulation of the same copy (tests/gpu_util.py assert_copy), the ring
  integers after every step, and the float32 checkpoint after the last fold
  within 1e-4 per head of the oracle state (page "ReplaySSM: Cache SSM
  Inputs, Not State", Abstract: a low-precision copy serves the outputs
  while the float32 checkpoint takes the updates);
* speculative verify (B=256, H=64, W=5, accepted drafts ~ U{0..5}), 32 fused
  rounds through replay_verify_step: every draft's output of every sequence
  within 1e-4 per head, the ring integers of every sequence after every
  round equal to the integer model's;
* a Gated DeltaNet layer (B=256, H=32, G=16, P=N=128, L=16, bf16 q/k/v,
  float32 checkpoint; the gated delta rule, oracle.core.eager_gdn), 48 steps
  (3 folds) through replay_step: every output of every sequence within 1e-4
  per head (the floor's term magnitude as in tests/test_gpu_gdn.py), every
  checkpoint after the last fold within 1e-4 of the oracle state.

Page "ReplaySSM: Cachear Inputs, No Estado", "Los dos caminos": the
output of a head is y_t = S_t q_t, and the rewriting changes no result.
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


def test_step_every_sequence_decode_workload():
    w = synth.named("decode")
    T, L = 64, w.ring_len
    gu.note(f"full batch: fused step {w} T={T}")
    dev = gu.DevInputsTorch(w, 0, T)
    layer = _layer(w)
    model = oring.RingModel(w.batch, L)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=L)
        model.append(1)
        model.flush(L)
        gu.check_ring(layer, model, f"step {t}")
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    S = np.zeros((w.batch, w.heads, w.head_dim, w.state_dim))
    y_ref = runs.standard(x, S)
    gu.assert_f32(y.cpu().numpy(), y_ref, gu.y_abs_standard(x, S.shape), what="all 256 sequences:")
    del y_ref
    # T is a multiple of L: the last step folded, so the checkpoint is the state after token T
    S_gpu = layer.s_master.cpu().numpy()
    e = runs.normwise_rel_err(S_gpu, S, axes=(-2, -1))
    print(f"  checkpoint per-head max {float(e.max()):.3e}", flush=True)
    assert float(e.max()) <= gu.TOL_F32
    layer.close()


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_copy_step_every_sequence_decode_workload(fmt):
    w = synth.named("decode")
    T, L = 32, w.ring_len
    gu.note(f"full batch: copy-mode step, {fmt} copy, {w} T={T}")
    dev = gu.DevInputsTorch(w, 0, T)
    layer = _layer(w, read_copy=fmt)
    model = oring.RingModel(w.batch, L)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=L)
        model.append(1)
        model.flush(L)
        gu.check_ring(layer, model, f"step {t}")
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    S = np.zeros((w.batch, w.heads, w.head_dim, w.state_dim))
    y_emul = runs.separated(x, S, L, fmt)   # S ends as the exact state after token T
    gu.assert_copy(y.cpu().numpy(), y_emul, fmt, "all 256 sequences:")
    del y_emul
    e = runs.normwise_rel_err(layer.s_master.cpu().numpy(), S, axes=(-2, -1))
    print(f"  checkpoint per-head max {float(e.max()):.3e}", flush=True)
    assert float(e.max()) <= gu.TOL_F32
    layer.close()


def test_verify_step_every_sequence_verify_workload():
    w = synth.named("verify")
    R, W = 32, 5
    gu.note(f"full batch: fused verify rounds {w} R={R} W={W}")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputsTorch(w, 0, R * W)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model, fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    S = np.zeros((w.batch, w.heads, w.head_dim, w.state_dim))
    y_ref = runs.verify_rounds(x, accept, W, S)                       # [R][W][B][H][P]
    y_abs = gu.y_abs_verify(x, accept, W, S.shape)
    gu.assert_f32(y.cpu().numpy().transpose(0, 2, 1, 3, 4), y_ref, y_abs, what="all 256 sequences:")
    layer.close()


class _GdnInputsTorch(gu.DevInputsTorch):
    """Gated DeltaNet inputs (synth.gdn_inputs_torch) generated on the device."""

    def __init__(self, w, t0, t1):
        self.w = w
        self.t0 = t0
        self.t = synth.gdn_inputs_torch(w, t0, t1, device=gu.DEV)


def test_step_every_sequence_gdn_workload():
    from tests import parity
    w = synth.named("gdn")
    T, L = 48, w.ring_len
    gu.note(f"full batch: gated delta rule {w} T={T}")
    dev = _GdnInputsTorch(w, 0, T)
    layer = _layer(w, rule="gdn")
    model = oring.RingModel(w.batch, L)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=L)
        model.append(1)
        model.flush(L)
    gu.check_ring(layer, model, "gated delta rule, last step")
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    S = np.zeros((w.batch, w.heads, w.head_dim, w.state_dim))
    y_ref = runs.standard(x, S, rule="gdn")
    y_abs = runs.standard(parity.abs_inputs(x), np.zeros_like(S), rule="ssd")
    gu.assert_f32(y.cpu().numpy(), y_ref, y_abs, what="all 256 sequences:")
    del y_ref, y_abs
    S_gpu = layer.s_master.cpu().numpy()
    e = runs.normwise_rel_err(S_gpu, S, axes=(-2, -1))
    print(f"  checkpoint per-head max {float(e.max()):.3e}", flush=True)
    assert float(e.max()) <= gu.TOL_F32
    layer.close()
