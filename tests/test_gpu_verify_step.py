"""The fused speculative-verify round (replay_verify_step) on the GPU: fold if
due, append the drafts, score them, in one launch.

- Bit for bit against the same rounds run as the flush, append and verify
  calls (outputs, checkpoints, pointers and every ring slot), over shapes
  with ragged groups, both routes (fold / no fold) mixed inside one launch,
  and the configurations that fall back to the calls; windows of 5 and more
  take the matrix cores in both (the same code and operands).
- Against the float64 oracle at the verify workload's full size (B=256,
  H=64, W=5, 128 rounds; sampled sequences) with the ring integers of all
  sequences checked after every round, and at small sizes on every sequence.
- Error paths: drafts that do not fit and a pointer at its limit leave the
  sequence unchanged, set its bit and give NaN outputs."""
import numpy as np
import pytest
import torch

import synth
from oracle import ring as oring
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL_F32 = 1e-4
RING = ("ring_q", "ring_k", "ring_v", "ring_dt", "ring_a")


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    layer = lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                            io_dtype=w.io_dtype, device=gu.DEV, **kw)
    for name in RING:   # defined contents, so whole rings can be compared
        layer.t[name].zero_()
    return layer


@pytest.mark.parametrize("P,N,io,L,W,B,H,G,rc", [
    (64, 128, "bf16", 16, 5, 6, 16, 4, None),     # the verify workload's head shape
    (64, 128, "bf16", 16, 8, 3, 8, 8, None),      # one head per group
    (64, 128, "bf16", 16, 4, 4, 8, 2, None),      # the register sums
    (16, 16, "bf16", 16, 6, 3, 4, 2, None),       # matrix cores, rows shorter than a cache line
    (128, 128, "bf16", 16, 7, 2, 8, 2, None),     # matrix cores, 8 streaming wavefronts
    (64, 64, "bf16", 12, 6, 4, 4, 2, None),       # matrix cores, 256-byte rows
    (16, 16, "bf16", 4, 3, 4, 6, 2, None),        # W close to L: folds most rounds
    (64, 64, "bf16", 8, 1, 5, 4, 2, None),
    (64, 64, "bf16", 9, 3, 4, 6, 3, None),        # register sums, two pieces of a row a lane
    (128, 128, "bf16", 12, 4, 2, 12, 3, None),
    (64, 128, "bf16", 5, 5, 3, 4, 1, None),       # W = L: every round folds
    (64, 128, "f32", 16, 5, 3, 8, 2, None),       # f32 io: the calls in turn
    (64, 128, "f32", 16, 12, 3, 8, 2, None),      # f32 io past 8: verify on the float32 matrix cores
    (64, 128, "bf16", 32, 6, 3, 8, 2, None),      # L > 16: the calls in turn
    (64, 128, "bf16", 16, 5, 3, 8, 2, "bf16"),    # a bf16 read copy: the calls in turn
    (64, 128, "bf16", 16, 5, 6, 16, 4, "fp8"),    # e4m3 copy: one launch (fold: master + copy rewrite)
    (64, 128, "bf16", 16, 5, 6, 16, 4, "fp4"),    # FP4 copy: one launch
    (64, 128, "bf16", 8, 3, 4, 8, 2, "fp8"),      # folds most rounds
    (64, 64, "bf16", 12, 4, 3, 4, 2, "fp4"),
    (64, 64, "bf16", 6, 2, 5, 6, 3, "fp8"),
    (16, 16, "bf16", 16, 5, 3, 4, 2, "fp4"),      # FP4 chunks of 2 bytes
    (16, 16, "bf16", 4, 3, 4, 6, 2, "fp8"),
    (64, 128, "bf16", 5, 5, 3, 4, 1, "fp4"),      # W = L: every round folds
    (64, 128, "bf16", 16, 7, 3, 8, 2, "fp8"),     # W past 5: the calls in turn
    (128, 128, "bf16", 16, 4, 2, 4, 2, "fp8"),    # 128 x 128: the calls in turn
])
def test_verify_step_equals_calls(P, N, io, L, W, B, H, G, rc):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=140 + P + L + W)
    R = 14
    gu.note(f"verify_step vs calls {w} W={W} copy={rc}")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    kw = {} if rc is None else {"read_copy": rc}
    fused, calls = _layer(w, **kw), _layer(w, **kw)
    y_f = gu.run_verify(fused, w, dev, R, W, accept, fused=True)
    y_c = gu.run_verify(calls, w, dev, R, W, accept)
    torch.cuda.synchronize()
    assert fused.get_error()[0] == 0 and calls.get_error()[0] == 0
    assert np.array_equal(y_f.cpu().numpy(), y_c.cpu().numpy())
    assert np.isfinite(y_f.cpu().numpy()).all()
    for name in ("s_master", "pos", "base") + RING:
        assert torch.equal(fused.t[name], calls.t[name]), name
    if rc is not None:
        assert torch.equal(fused.t["s_copy"], calls.t["s_copy"])
        if fused.t["s_scale"] is not None:
            assert torch.equal(fused.t["s_scale"], calls.t["s_scale"])
    fused.close()
    calls.close()


@pytest.mark.parametrize("P,N,io,L,W,B,H,G,rc,bad", [
    (64, 128, "bf16", 16, 5, 6, 16, 4, None, False),   # the float32 round: one launch
    (64, 128, "bf16", 16, 5, 6, 16, 4, None, True),    # with an out-of-range rollback
    (128, 128, "bf16", 12, 4, 2, 12, 3, None, False),
    (64, 128, "bf16", 16, 5, 6, 16, 4, "fp8", True),   # e4m3 copy: one launch
    (64, 64, "bf16", 12, 4, 3, 4, 2, "fp4", False),    # FP4 copy: one launch
    (64, 128, "bf16", 16, 5, 3, 8, 2, "bf16", True),   # bf16 copy: rollback kernel, then the calls
    (64, 128, "bf16", 32, 6, 3, 8, 2, None, False),    # L > 16: rollback kernel, then the calls
])
def test_rollback_verify_step_equals_calls(P, N, io, L, W, B, H, G, rc, bad):
    """replay_rollback_verify_step(n_reject of round r-1, round r) equals
    replay_rollback then the round's three calls, bit for bit: outputs,
    checkpoint, copy and scales, pointers, ring slots and error bits (with
    bad=True one sequence's rollback is out of range in one round: flagged,
    its pointer kept, the round run); pointers checked against the ring
    model after every launch."""
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=170 + P + L + W)
    R = 12
    gu.note(f"rollback_verify_step vs calls {w} W={W} copy={rc} bad={bad}")
    accept = synth.accept_counts(w, R, W)
    nrej = (W - accept).astype(np.int32)
    if bad:
        nrej[4, 1] = L + 1   # more than any count
    dev = gu.DevInputs(w, 0, R * W)
    kw = {} if rc is None else {"read_copy": rc}
    fused, calls = _layer(w, **kw), _layer(w, **kw)
    model = oring.RingModel(w.batch, w.ring_len)
    y_f = gu.run_verify(fused, w, dev, R, W, accept, model=model, rollback_fused=True, nrej=nrej)
    y_c = gu.run_verify(calls, w, dev, R, W, accept, nrej=nrej)
    torch.cuda.synchronize()
    e_f, s_f = fused.get_error()
    e_c, s_c = calls.get_error()
    assert e_f == e_c and np.array_equal(np.asarray(s_f), np.asarray(s_c))
    assert (e_f != 0) == bad
    assert np.array_equal(y_f.cpu().numpy(), y_c.cpu().numpy())
    for name in ("s_master", "pos", "base") + RING:
        if fused.t[name] is not None:
            assert torch.equal(fused.t[name], calls.t[name]), name
    if rc is not None:
        assert torch.equal(fused.t["s_copy"], calls.t["s_copy"])
        if fused.t["s_scale"] is not None:
            assert torch.equal(fused.t["s_scale"], calls.t["s_scale"])
    fused.close()
    calls.close()


def test_verify_step_workload():
    """B=256 H=64 G=8 P=64 N=128 L=16, W=5, accepted drafts ~ Uniform{0..5},
    128 fused rounds (the launch sequence bench.py times); 6 sampled
    sequences against the oracle, ring integers of all 256 after every round."""
    w = synth.named("verify")
    R, W, seqs = 128, 5, [0, 3, 100, 128, 254, 255]
    gu.note("verify_step workload")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model, fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, R * W, seqs)
    S = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_ref = runs.verify_rounds(x, accept[:, seqs], W, S)
    y_gpu = y.cpu().numpy()[:, seqs].transpose(0, 2, 1, 3, 4)
    gu.assert_f32(y_gpu, y_ref, gu.y_abs_verify(x, accept[:, seqs], W, S.shape))
    layer.close()


@pytest.mark.parametrize("P,N,L,W,B,H,G", [(16, 16, 6, 4, 3, 4, 2), (64, 128, 16, 7, 4, 8, 4),
                                           (128, 128, 9, 2, 2, 6, 3)])
def test_verify_step_small_all_sequences(P, N, L, W, B, H, G):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=170 + P + L + W)
    R = 16
    gu.note(f"verify_step oracle {w} W={W}")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model, fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    seqs = list(range(B))
    x = gu.oracle_inputs(w, 0, R * W, seqs)
    S = np.zeros((B, H, P, N))
    y_ref = runs.verify_rounds(x, accept, W, S)
    gu.assert_f32(y.cpu().numpy().transpose(0, 2, 1, 3, 4), y_ref, gu.y_abs_verify(x, accept, W, S.shape))
    layer.close()


def test_verify_step_errors():
    """flush_at above L-W+1: the third round's drafts do not fit (RING_OVERFLOW);
    a pointer at 2^31-3 cannot take 3 drafts (POS_OVERFLOW).  Those sequences
    keep pointers and rings and get NaN outputs; the others are unaffected
    (equal to the calls run on them alone)."""
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=4, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=8,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=191)
    W = 3
    gu.note("verify_step errors")
    dev = gu.DevInputs(w, 0, 4 * W)
    layer = _layer(w)
    ref = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    # rounds 0, 1 accept everything; with flush_at = L + 1 nothing folds
    y = torch.zeros((3, w.batch, W, w.heads, 64), dtype=torch.float32, device=gu.DEV)
    for rd in range(2):
        layer.verify_step(W, *dev.window(rd * W, W), y[rd], flush_at=w.ring_len + 1)
        model.append(W)
    gu.check_ring(layer, model, "two rounds")
    # sequence 2: pointer near the limit (empty ring there)
    layer.pos[2] = layer.base[2] = model.pos[2] = model.base[2] = 2 ** 31 - 3
    before = {n: layer.t[n].clone() for n in ("s_master",) + RING}
    layer.verify_step(W, *dev.window(2 * W, W), y[2], flush_at=w.ring_len + 1)
    torch.cuda.synchronize()
    word, per = layer.get_error()
    # sequences 0, 1, 3 hold 6 entries: 6 + 3 > 8
    assert per == [lad.SEQERR_RING_OVERFLOW, lad.SEQERR_RING_OVERFLOW, lad.SEQERR_POS_OVERFLOW,
                   lad.SEQERR_RING_OVERFLOW], per
    gu.check_ring(layer, model, "failed round")
    assert np.isnan(y[2].cpu().numpy()).all()
    for n, t in before.items():
        assert torch.equal(layer.t[n], t), n
    # a fold then makes room: flush_at = L - W + 1 folds the 6 entries
    y3 = torch.zeros((w.batch, W, w.heads, 64), dtype=torch.float32, device=gu.DEV)
    layer.verify_step(W, *dev.window(3 * W, W), y3)
    torch.cuda.synchronize()
    word, per = layer.get_error()
    assert per == [0, 0, lad.SEQERR_POS_OVERFLOW, 0], per
    y3c = y3.cpu().numpy()
    assert np.isfinite(y3c[[0, 1, 3]]).all() and np.isnan(y3c[2]).all()
    # the same rounds as calls on a fresh layer (sequences 0, 1, 3)
    yr = torch.zeros((w.batch, W, w.heads, 64), dtype=torch.float32, device=gu.DEV)
    for rd in range(2):
        ref.append(W, *dev.window(rd * W, W))
        ref.verify(W, yr)
    assert np.array_equal(y[1].cpu().numpy(), yr.cpu().numpy())
    ref.flush(w.ring_len - W + 1)
    ref.append(W, *dev.window(3 * W, W))
    ref.verify(W, yr)
    torch.cuda.synchronize()
    assert np.array_equal(y3c[[0, 1, 3]], yr.cpu().numpy()[[0, 1, 3]])
    assert torch.equal(layer.s_master[[0, 1, 3]], ref.s_master[[0, 1, 3]])
    layer.close()
    ref.close()


@pytest.mark.parametrize("copy", ["fp8", "fp4"])
def test_verify_step_copy_workload(copy):
    """B=256 H=64 G=8 P=64 N=128 L=16, W=5, accepts ~ U{0..5}, 32 fused rounds
    with an e4m3 / FP4 read copy (one launch a round): 16 sequences spread
    over the batch against the oracle's emulation of rounds read from that
    copy (tests/gpu_util.py assert_copy), ring integers of all 256 after every round."""
    w = synth.named("verify")
    R, W = 32, 5
    gu.note(f"verify_step copy workload {copy}")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputsTorch(w, 0, R * W)
    layer = _layer(w, read_copy=copy)
    model = oring.RingModel(w.batch, w.ring_len)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model, fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    seqs = list(range(0, w.batch, 16))
    x = dev.oracle(seqs)
    S0 = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_emul = runs.verify_rounds_copy(x, accept[:, seqs], W, S0, w.ring_len, copy)
    gu.assert_copy(y.cpu().numpy()[:, seqs].transpose(0, 2, 1, 3, 4), y_emul, copy)
    layer.close()
