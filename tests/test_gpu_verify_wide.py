"""Speculative verify on the matrix cores (replay_verify from W = 6 on, up
to 16, with bf16 io; from W = 9 on with float32 io).

- Rounds of W drafts with rollback and flushes when the next window would
  not fit, against the float64 oracle (per token over the layer output:
  1e-4 per head for a float32 checkpoint; bf16 / e4m3 / MX FP4 copies against the oracle's
  emulation of the same copy, tests/gpu_util.py assert_copy) and the integer ring model.
- The same state scored with W = 16 here and W = 4 by the register kernel:
  the newest four positions agree to float32 rounding (the two kernels share
  nothing but the ring term's code).
- Float32 io past W = 8: the same rounds with float32 queries on the
  float32 matrix cores.
- Errors: count < W gives NaN and TOO_FEW; windows past 16 are rejected."""
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


@pytest.mark.parametrize("P,N,L,W,B,H,G,copy", [
    (64, 128, 16, 16, 3, 8, 2, None),      # the verify workload's head, W = L
    (64, 128, 16, 12, 4, 16, 4, None),
    (64, 64, 20, 9, 3, 4, 2, None),        # two ring blocks
    (128, 128, 32, 16, 2, 4, 2, None),
    (16, 16, 16, 11, 3, 6, 3, None),
    (64, 128, 16, 16, 3, 8, 2, "bf16"),
    (64, 128, 16, 10, 3, 8, 2, "fp8"),
    (16, 16, 16, 16, 2, 4, 1, "fp8"),      # e4m3 tile widened (N < 32)
    (64, 128, 16, 6, 3, 8, 2, None),       # the smallest window on the matrix cores
    (64, 128, 8, 8, 2, 8, 2, "bf16"),
    (128, 128, 16, 9, 2, 4, 2, "fp8"),
    (64, 64, 16, 7, 3, 4, 2, "bf16"),
    (64, 128, 16, 16, 3, 8, 2, "fp4"),      # one product per MX block
    (64, 64, 16, 9, 3, 4, 2, "fp4"),
    (128, 128, 32, 12, 2, 4, 2, "fp4"),
    (16, 16, 16, 13, 2, 4, 1, "fp4"),       # FP4 tile widened with its block scales (N < 32)
    (64, 128, 8, 6, 2, 8, 2, "fp4"),
])
def test_wide_verify_rounds(P, N, L, W, B, H, G, copy, io="bf16"):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=300 + P + L + W)
    R = 10
    gu.note(f"wide verify {w} W={W} copy={copy}")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    layer = _layer(w, **({} if copy is None else {"read_copy": copy}))
    model = oring.RingModel(B, L)
    y = gu.run_verify(layer, w, dev, R, W, accept, model=model)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, R * W, list(range(B)))
    S0 = np.zeros((B, H, P, N))
    if copy is None:
        y_ref, tol = runs.verify_rounds(x, accept, W, S0), 1e-4
    else:
        y_ref, tol = runs.verify_rounds_copy(x, accept, W, S0, L, copy), None
    if copy is None:
        gu.assert_f32(y.cpu().numpy().transpose(0, 2, 1, 3, 4), y_ref, gu.y_abs_verify(x, accept, W, S0.shape))
    else:
        gu.assert_copy(y.cpu().numpy().transpose(0, 2, 1, 3, 4), y_ref, copy)
    layer.close()


@pytest.mark.parametrize("P,N,L,W,B,H,G,copy", [
    (64, 128, 16, 16, 3, 8, 2, None),      # the verify workload's head, W = L
    (64, 64, 20, 9, 3, 4, 2, None),        # two ring blocks
    (128, 128, 32, 12, 2, 4, 2, None),
    (16, 16, 16, 11, 3, 6, 3, None),       # N < 32: half the dot columns masked
    (64, 128, 16, 10, 3, 8, 2, "bf16"),
    (64, 128, 16, 12, 3, 8, 2, "fp8"),
    (16, 16, 16, 16, 2, 4, 1, "fp8"),
    (64, 128, 16, 16, 3, 8, 2, "fp4"),
    (128, 128, 16, 9, 2, 4, 2, "fp4"),
    (16, 16, 16, 14, 2, 4, 1, "fp4"),
])
def test_wide_verify_rounds_f32_io(P, N, L, W, B, H, G, copy):
    """Float32 io past the register kernel's 8: the queries stay float32 and
    every product runs on the float32 matrix cores."""
    test_wide_verify_rounds(P, N, L, W, B, H, G, copy, io="f32")


@pytest.mark.parametrize("P,N,copy,io", [(64, 128, None, "bf16"), (128, 128, None, "bf16"), (64, 128, "fp8", "bf16"),
                                         (64, 128, "fp4", "bf16"), (64, 128, None, "f32"), (64, 64, "fp4", "f32")])
def test_wide_window_agrees_with_register_kernel(P, N, copy, io):
    """16 entries in the ring: verify(16) on the matrix cores and verify(4) in
    registers score the newest four positions of the same state."""
    w = synth.Workload(batch=3, heads=8, groups=2, head_dim=P, state_dim=N, ring_len=16, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=330 + P)
    gu.note(f"wide vs register verify P={P} N={N} copy={copy} io={io}")
    dev = gu.DevInputs(w, 0, 40)
    layer = _layer(w, **({} if copy is None else {"read_copy": copy}))
    for t in range(24):                        # a non-zero checkpoint first
        layer.append(1, *dev.step(t))
        layer.flush(16)
    layer.flush(1)                             # empty ring, then a full one
    layer.append(16, *dev.window(24, 16))
    y16 = torch.empty((3, 16, 8, P), dtype=torch.float32, device=gu.DEV)
    y4 = torch.empty((3, 4, 8, P), dtype=torch.float32, device=gu.DEV)
    layer.verify(16, y16)
    layer.verify(4, y4)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    tok, _, _ = gu.errors(y16[:, 12:].cpu().numpy(), y4.cpu().numpy().astype(np.float64))
    assert tok <= 1e-5, tok
    layer.close()


def test_wide_verify_errors():
    import linear_attention_decode_amd as lad
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=16, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=341)
    gu.note("wide verify errors")
    dev = gu.DevInputs(w, 0, 12)
    layer = _layer(w)
    layer.append(12, *dev.window(0, 12))
    y = torch.zeros((3, 13, 4, 64), dtype=torch.float32, device=gu.DEV)
    layer.verify(13, y)                        # 12 entries < 13: every sequence fails
    torch.cuda.synchronize()
    word, per = layer.get_error()
    assert per == [lad.SEQERR_TOO_FEW] * 3
    assert torch.isnan(y).all()
    y12 = torch.zeros((3, 12, 4, 64), dtype=torch.float32, device=gu.DEV)
    layer.verify(12, y12)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0 and torch.isfinite(y12).all()
    with pytest.raises(lad.ReplayError):
        layer.verify(17, torch.zeros((3, 17, 4, 64), dtype=torch.float32, device=gu.DEV))
    layer.close()
    lay = lad.ReplayLayer(2, 4, 2, 64, 128, 16, io_dtype="f32", device=gu.DEV)
    with pytest.raises(lad.ReplayError):
        lay.verify(17, torch.zeros((2, 17, 4, 64), dtype=torch.float32, device=gu.DEV))
    lay.close()
