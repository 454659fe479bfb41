"""Speculative verify on the GPU: rounds of W drafts scored against one
checkpoint read, rollback by moving the ring pointer, flushes when the next
window would not fit -- against the float64 oracle (which replays the
accepted prefix of every round with the eager recurrence) and the integer
ring model.  Tolerance as for decode (float32 checkpoint, 1e-4 per head)."""
import numpy as np
import pytest
import torch

import synth
from oracle import ring as oring
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL_F32 = 1e-4


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    return lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                           io_dtype=w.io_dtype, device=gu.DEV, **kw)


def _verify_case(w, R, W, seqs, accept=None):
    gu.note(f"verify {w} R={R} W={W}")
    if accept is None:
        accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, R * W, seqs)
    S = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_ref = runs.verify_rounds(x, accept[:, seqs], W, S)          # [R][W][b][H][P]
    y_gpu = y.cpu().numpy()[:, seqs].transpose(0, 2, 1, 3, 4)      # [R][W][b][H][P]
    gu.assert_f32(y_gpu, y_ref, gu.y_abs_verify(x, accept[:, seqs], W, S.shape))
    layer.close()
    return y, accept


def test_verify_workload():
    """Speculative verify: B=256 H=64 G=8 P=64 N=128 L=16, W=5 drafts per
    round, accepted drafts ~ Uniform{0..5}, 128 rounds; 6 sampled sequences
    against the oracle, ring integers of all 256 after every call."""
    w = synth.named("verify")
    _verify_case(w, 128, 5, [0, 3, 100, 128, 254, 255])


@pytest.mark.parametrize("P,N,io,L,W,B,H,G", [
    (16, 16, "f32", 5, 3, 3, 6, 2),
    (16, 16, "f32", 4, 4, 2, 4, 1),
    (64, 64, "bf16", 8, 8, 3, 4, 2),
    (64, 128, "bf16", 6, 2, 5, 8, 8),
    (64, 128, "f32", 32, 7, 2, 16, 4),
    (128, 128, "bf16", 9, 6, 2, 4, 2),
    (64, 128, "bf16", 3, 1, 4, 16, 8),
    # register sums with several pieces of a row a lane: 64-column rows (two
    # pieces), 128 x 128 tiles (512 streaming threads), float32 io
    (64, 64, "bf16", 8, 3, 3, 4, 2),
    (64, 64, "f32", 9, 5, 2, 6, 3),
    (128, 128, "bf16", 8, 4, 2, 4, 2),
    (128, 128, "f32", 7, 2, 3, 2, 1),
])
def test_verify_ragged(P, N, io, L, W, B, H, G):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L,
                       io_dtype=io, config=synth.CONFIG_ID["misc"], layer=100 + P + L + W)
    _verify_case(w, 12, W, list(range(B)))


def test_rollback_equals_accepted_prefix_replay():
    """After speculative rounds with rejections, the state (flushed to the
    checkpoint) equals the state of a plain decode run fed only the accepted
    drafts, and every accepted draft's output equals that run's output."""
    w = synth.Workload(batch=8, heads=16, groups=4, head_dim=64, state_dim=128, ring_len=16,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=41)
    R, W = 20, 4
    accept = synth.accept_counts(w, R, W)
    gu.note("rollback vs prefix replay")
    dev = gu.DevInputs(w, 0, R * W)
    lay_v = _layer(w)
    y_v = gu.run_verify(lay_v, w, dev, R, W, accept)
    lay_v.flush(1)
    torch.cuda.synchronize()
    for b in range(w.batch):
        keep = [r * W + i for r in range(R) for i in range(accept[r, b])]
        if not keep:
            continue
        # replay: this sequence's accepted tokens only, as plain decode (B=1 layer)
        w1 = synth.Workload(batch=1, heads=w.heads, groups=w.groups, head_dim=64, state_dim=128,
                            ring_len=w.ring_len, io_dtype="bf16")
        lay_1 = _layer(w1)
        yb = torch.empty((len(keep), 1, w.heads, 64), dtype=torch.float32, device=gu.DEV)
        for n, t in enumerate(keep):
            q, k, v, dt, a = (x[b:b + 1] for x in dev.step(t))
            lay_1.append(1, q, k, v, dt, a)
            lay_1.decode(yb[n])
            lay_1.flush(w.ring_len)
        lay_1.flush(1)
        torch.cuda.synchronize()
        S_v = lay_v.s_master[b].cpu().numpy().astype(np.float64)
        S_1 = lay_1.s_master[0].cpu().numpy().astype(np.float64)
        e = runs.normwise_rel_err(S_v, S_1, axes=(-3, -2, -1))
        assert float(e) <= 1e-5, (b, float(e))
        # outputs of the accepted drafts
        yv = y_v.cpu().numpy()[:, b]                                  # [R][W][H][P]
        acc_out = np.stack([yv[r, i] for r in range(R) for i in range(accept[r, b])])
        e = runs.normwise_rel_err(acc_out, yb.cpu().numpy()[:, 0])
        assert float(np.max(e)) <= 1e-5, (b, float(np.max(e)))
        lay_1.close()
    lay_v.close()
