"""Gated DeltaNet layers on the GPU (replay_config.rule = GATED_DELTA),
against the float64 gated-delta-rule oracle (core.eager_gdn, pinned by
tests/test_oracle_gdn.py).

- Standard decode through replay_step (append, the output-only route --
  backward chain over the ring, one pass over S0 -- and the fold when the
  ring is full), ragged shapes, both io dtypes, rings of 16 and 32 entries,
  from a non-zero checkpoint; the checkpoint after a final fold against the
  oracle's state.
- Speculative rounds with rollback, by separate calls and by
  replay_verify_step (the same kernels: equal bit for bit): W = 1..8 (register
  sums) and W = 9..16 (S0 W_0^T on the matrix cores).
- The eager step of this layer (replay_eager_step) against the oracle.
- Low-precision copies (bf16, e4m3, MX FP4), separated and shared: outputs
  against the oracle's emulation of the same copy (oracle.runs.separated /
  shared / verify_rounds_copy with the gated delta rule), and, separated,
  the copy's codes and scales against the oracle's quantisers applied to the
  float32 checkpoint the same flush wrote, bit for bit.
- The Gated DeltaNet workload's shapes (B=256, H=32, G=16, P=N=128, L=16,
  bf16), 64 steps, sampled sequences across the batch.
- Errors: windows past 16 are rejected, count < W gives NaN and TOO_FEW.

Metric: the float32 per-head metric of tests/parity.py (1e-4).  Its
conditioning floor takes as term magnitude the Mamba-2 recurrence run on
|q|, |k|, |v| and |S0| with beta as dt and alpha as a: the decayed sum of
every write's magnitude (the delta rule's own erase terms only shrink a
state whose keys have unit length, so they add no magnitude of their own).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ring as oring
from oracle import runs
from tests import gpu_util as gu
from tests import parity

pytestmark = pytest.mark.gpu


class DevGdn:
    """gdn_inputs of tokens t0..t1-1, on the device, in the layouts of gu.DevInputs."""

    def __init__(self, w, t0, t1, seqs=None):
        self.w, self.t0 = w, t0
        self.host = synth.gdn_inputs(w, t0, t1, seqs=seqs)
        self.t = {k: gu.to_dev(v) for k, v in self.host.items()}

    def step(self, t):
        i = t - self.t0
        return tuple(self.t[n][i] for n in ("q", "k", "v", "dt", "a"))

    def window(self, t, W):
        i = t - self.t0
        return tuple(self.t[n][i:i + W].transpose(0, 1).contiguous() for n in ("q", "k", "v", "dt", "a"))

    def oracle(self, seqs=None):
        pick = (lambda v: v) if seqs is None else (lambda v: v[:, seqs])
        return runs.widen_inputs({k: pick(v) for k, v in self.host.items()}, self.w.io_dtype)


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    return lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                           io_dtype=w.io_dtype, device=gu.DEV, rule="gdn", **kw)


def _y_abs(x, S0):
    return runs.standard(parity.abs_inputs(x), np.abs(S0).astype(np.float64), rule="ssd")


@pytest.mark.parametrize("P,N,H,G,L,io,B", [
    (16, 16, 4, 2, 4, "f32", 3),
    (64, 64, 4, 2, 5, "bf16", 3),
    (64, 128, 8, 4, 8, "bf16", 2),
    (128, 128, 4, 2, 16, "bf16", 2),
    (128, 128, 4, 4, 32, "f32", 2),      # two ring blocks: 32-entry chain
    (64, 128, 6, 3, 16, "f32", 3),
])
def test_gdn_decode_ragged(P, N, H, G, L, io, B):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=400 + P + L)
    T = 3 * L + 2
    gu.note(f"gdn decode {w}")
    S0 = synth.checkpoint_state(w, scale=0.5)
    dev = DevGdn(w, 0, T)
    layer = _layer(w)
    layer.load_checkpoint(gu.to_dev(S0))
    model = oring.RingModel(B, L)
    y = torch.empty((T, B, H, P), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=L)
        model.append(1)
        model.flush(L)
    layer.flush(1)                        # fold what is left: the checkpoint is S_T
    model.flush(1)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    gu.check_ring(layer, model, "gdn decode")
    x = dev.oracle()
    S = S0.astype(np.float64).copy()
    y_ref = runs.standard(x, S, rule="gdn")
    gu.assert_f32(y.cpu().numpy(), y_ref, _y_abs(x, S0), what=f"gdn P={P} N={N} L={L}")
    Sg = layer.s_master.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(Sg - S)) / np.max(np.abs(S))
    print(f"  checkpoint after the last fold: max rel {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("P,N,L,W,B,H,G", [
    (64, 128, 16, 5, 3, 8, 2),
    (128, 128, 16, 8, 2, 4, 2),
    (16, 16, 8, 3, 3, 4, 1),
    (64, 64, 32, 4, 2, 4, 2),
    (64, 128, 16, 1, 3, 4, 2),
    (64, 128, 16, 12, 3, 4, 2),            # matrix cores from here on
    (128, 128, 16, 16, 2, 4, 2),
    (16, 16, 16, 9, 3, 4, 1),
    (64, 64, 32, 13, 2, 4, 2),
])
def test_gdn_verify_rounds(P, N, L, W, B, H, G):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=420 + P + L + W)
    R = 12
    gu.note(f"gdn verify {w} W={W}")
    accept = synth.accept_counts(w, R, W)
    dev = DevGdn(w, 0, R * W)
    layer = _layer(w)
    model = oring.RingModel(B, L)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model)
    twin = _layer(w)
    y_fused = gu.run_verify(twin, w, dev, R, W, accept, fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0 and twin.get_error()[0] == 0
    assert torch.equal(y, y_fused)                              # replay_verify_step: the same kernels
    assert torch.equal(layer.s_master, twin.s_master)
    x = dev.oracle()
    S0 = np.zeros((B, H, P, N))
    y_ref = runs.verify_rounds(x, accept, W, S0.copy(), rule="gdn")
    y_abs = runs.verify_rounds(parity.abs_inputs(x), accept, W, S0.copy(), rule="ssd")
    gu.assert_f32(y.cpu().numpy().transpose(0, 2, 1, 3, 4), y_ref, y_abs, what=f"gdn verify W={W}")


@pytest.mark.parametrize("P,N,io", [(64, 128, "bf16"), (128, 128, "f32"), (16, 16, "bf16")])
def test_gdn_eager_step(P, N, io):
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=P, state_dim=N, ring_len=4, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=440 + P)
    T = 5
    gu.note(f"gdn eager {w}")
    S0 = synth.checkpoint_state(w, scale=0.5)
    dev = DevGdn(w, 0, T)
    cfg = lad.ReplayConfig(w.batch, w.heads, w.groups, P, N, w.ring_len, lad._DTYPE_CODE[io], lad.NONE, 0,
                           lad.GATED_DELTA)
    s_a = gu.to_dev(S0)
    s_b = torch.empty_like(s_a)
    y = torch.empty((T, w.batch, w.heads, P), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        lad.replay_eager_step(cfg, s_a, s_b, *dev.step(t), y[t])
        s_a, s_b = s_b, s_a
    torch.cuda.synchronize()
    x = dev.oracle()
    S = S0.astype(np.float64).copy()
    y_ref = runs.standard(x, S, rule="gdn")
    gu.assert_f32(y.cpu().numpy(), y_ref, _y_abs(x, S0), what=f"gdn eager P={P}")
    assert np.max(np.abs(s_a.cpu().numpy() - S)) <= 1e-4 * np.max(np.abs(S))


def test_gdn_workload_sampled():
    """The Gated DeltaNet workload (B=256, H=32, G=16, P=N=128, L=16, bf16),
    64 steps through replay_step from a zero checkpoint; 8 sequences across
    the batch against the oracle, the ring integers of all 256."""
    w = synth.named("gdn")
    T, seqs = 64, [0, 37, 100, 127, 128, 200, 254, 255]
    gu.note("gdn workload")
    dev = DevGdn(w, 0, T)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=w.ring_len)
        model.append(1)
        model.flush(w.ring_len)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    gu.check_ring(layer, model, "gdn workload")
    x = dev.oracle(seqs)
    S0 = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_ref = runs.standard(x, S0.copy(), rule="gdn")
    gu.assert_f32(y.cpu().numpy()[:, seqs], y_ref, _y_abs(x, S0), what="gdn workload")


def test_gdn_errors():
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=16, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=450)
    gu.note("gdn errors")
    dev = DevGdn(w, 0, 12)
    layer = _layer(w)
    layer.append(4, *dev.window(0, 4))
    y = torch.zeros((3, 5, 4, 64), dtype=torch.float32, device=gu.DEV)
    layer.verify(5, y)                      # 4 entries < 5: every sequence fails
    torch.cuda.synchronize()
    word, per = layer.get_error()
    assert per == [lad.SEQERR_TOO_FEW] * 3
    assert torch.isnan(y).all()
    layer.append(8, *dev.window(4, 8))
    with pytest.raises(lad.ReplayError):
        layer.verify(17, torch.zeros((3, 17, 4, 64), dtype=torch.float32, device=gu.DEV))
    y12 = torch.zeros((3, 12, 4, 64), dtype=torch.float32, device=gu.DEV)
    layer.verify(12, y12)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0 and torch.isfinite(y12).all()
    layer.close()


def _check_codes(layer, fmt):
    """The copy equals the oracle's quantisers applied to the float32 checkpoint, bit for bit."""
    import oracle
    S = layer.s_master.cpu().numpy()
    if fmt == "bf16":
        got = layer.s_copy.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, oracle.bf16_encode(S))
    elif fmt == "fp8":
        codes, scale = oracle.quant_heads_e4m3(S)
        assert np.array_equal(layer.s_scale.cpu().numpy(), scale)
        assert np.array_equal(layer.s_copy.cpu().numpy(), codes)
    else:
        packed, scale = oracle.core.quant_blocks_mxfp4(S)
        assert np.array_equal(layer.s_scale.cpu().numpy().reshape(scale.shape), scale)
        assert np.array_equal(layer.s_copy.cpu().numpy().reshape(packed.shape), packed)


COPIES = [(f, sh, P, N) for f in ("bf16", "fp8", "fp4") for sh in (False, True)
          for P, N in ((64, 128), (128, 128))] + [("fp4", False, 16, 16), ("fp8", True, 64, 64)]


@pytest.mark.parametrize("fmt,shared,P,N", COPIES,
                         ids=[f"{f}-{'shared' if sh else 'separated'}-{P}x{N}" for f, sh, P, N in COPIES])
def test_gdn_copy_decode(fmt, shared, P, N):
    """Standard decode through replay_step reading a bf16 / e4m3 / FP4 copy
    (L = 8, 3L + 2 steps from a non-zero checkpoint loaded through the copy's
    quantisers), against the oracle's emulation of the same copy."""
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=P, state_dim=N, ring_len=8, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=460 + P + N)
    T = 3 * w.ring_len + 2
    gu.note(f"gdn copy decode {fmt} shared={shared} {w}")
    S0 = synth.checkpoint_state(w, scale=0.5)
    dev = DevGdn(w, 0, T)
    layer = _layer(w, read_copy=fmt, shared_lowp=shared)
    layer.load_checkpoint(gu.to_dev(S0))
    y = torch.empty((T, w.batch, w.heads, P), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(*dev.step(t), y[t], flush_at=w.ring_len)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    S = S0.astype(np.float64).copy()
    emul = (runs.shared if shared else runs.separated)(x, S, w.ring_len, fmt, rule="gdn")
    gu.assert_copy(y.cpu().numpy(), emul, fmt, what=f"gdn {fmt} shared={shared} P={P} N={N}")
    if not shared:
        _check_codes(layer, fmt)
    layer.close()


@pytest.mark.parametrize("fmt,W", [("bf16", 4), ("fp8", 4), ("fp4", 4), ("fp8", 12), ("fp4", 16), ("bf16", 10)])
def test_gdn_copy_verify_rounds(fmt, W):
    """Speculative rounds (rollback) reading a copy, separated, by
    replay_verify_step, against the oracle's emulation of the copy; windows
    past 8 on the matrix cores."""
    L = 8 if W <= 4 else 16
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=L, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=470 + W)
    R = 10
    gu.note(f"gdn copy verify {fmt} {w}")
    accept = synth.accept_counts(w, R, W)
    dev = DevGdn(w, 0, R * W)
    layer = _layer(w, read_copy=fmt)
    y = gu.run_verify(layer, w, dev, R, W, accept, fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    emul = runs.verify_rounds_copy(x, accept, W, np.zeros((w.batch, w.heads, 64, 128)), w.ring_len, fmt, rule="gdn")
    gu.assert_copy(y.cpu().numpy().transpose(0, 2, 1, 3, 4), emul, fmt, what=f"gdn verify {fmt}")
    _check_codes(layer, fmt)
    layer.close()


@pytest.mark.parametrize("fmt", [None, "fp8", "fp4", "bf16"])
def test_gdn_wide_agrees_with_register_windows(fmt):
    """The same state scored with W = 16 and W = 8 (matrix cores) and W = 1
    (register sums): the positions the windows share agree to 1e-5 per token
    (the copies: the same codes read by both).  Slow decay (dt x 0.01), so
    that S0's part of the outputs stays large for the late positions."""
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=128, state_dim=128, ring_len=16, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=480, dt_scale=0.01)
    gu.note(f"gdn wide vs register windows {fmt}")
    S0 = synth.checkpoint_state(w, scale=0.5)
    dev = DevGdn(w, 0, 16)
    layer = _layer(w, read_copy=fmt)
    layer.load_checkpoint(gu.to_dev(S0))
    layer.append(16, *dev.window(0, 16))
    ys = {}
    for W in (16, 8, 1):
        ys[W] = torch.empty((3, W, 4, 128), dtype=torch.float32, device=gu.DEV)
        layer.verify(W, ys[W])
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = dev.oracle()
    S = S0.astype(np.float64).copy()
    y_ref = runs.standard(x, S, rule="gdn").transpose(1, 0, 2, 3)     # [B][16][H][P]
    e_s0 = runs.normwise_rel_err(runs.standard(x, np.zeros_like(S), rule="gdn").transpose(1, 0, 2, 3), y_ref)
    print(f"  S0's share of the outputs: per-token min {float(e_s0.min()):.3e}", flush=True)
    assert float(e_s0.min()) > 1e-3                   # S0 enters every position's output
    for W in (8, 1):
        e = runs.normwise_rel_err(ys[16][:, 16 - W:].cpu().numpy(), ys[W].cpu().numpy().astype(np.float64))
        print(f"  W=16 against W={W}: per-token max {float(e.max()):.3e}", flush=True)
        assert float(e.max()) <= 1e-5
    layer.close()
