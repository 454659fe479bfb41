"""Standard decode on the GPU (append -> output-only decode -> flush every
L steps) against the float64 oracle, through the C ABI.

Tolerance: the stated 1e-4 maximum relative error for a float32
checkpoint, per head: max_p |y - y_ref| / max_p |y_ref| for every
(sequence, token, head), the denominator floored at 1 % of the head's term
magnitude (tests/parity.py); the per-token figure over the layer's whole
output (heads x P) must meet it too.  Ring integers (pos, base) must match the integer model
bit for bit after every call.
"""
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


def _standard_case(w, T, seqs):
    gu.note(f"standard decode {w} T={T}")
    dev = gu.DevInputs(w, 0, T)
    layer = _layer(w)
    model = oring.RingModel(w.batch, w.ring_len)
    y = gu.run_standard(layer, w, dev, 0, T, model=model)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, T, seqs)
    S = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_ref = runs.standard(x, S)
    y_gpu = y.cpu().numpy()[:, seqs]
    gu.assert_f32(y_gpu, y_ref, gu.y_abs_standard(x, S.shape))
    # the checkpoint after the last flush equals the oracle state there
    last_flush = (T // w.ring_len) * w.ring_len
    if last_flush > 0:
        S_ref = np.zeros_like(S)
        runs.standard({k: v[:last_flush] for k, v in x.items()}, S_ref)
        S_gpu = layer.s_master.cpu().numpy()[seqs].astype(np.float64)
        e = runs.normwise_rel_err(S_gpu, S_ref, axes=(-3, -2, -1))
        assert float(e.max()) <= TOL_F32, float(e.max())
    layer.close()


def test_tiny_workload():
    """B=1 H=4 G=1 P=N=16 L=4, float32, 32 steps, flush every 4 steps."""
    _standard_case(synth.named("tiny"), 32, [0])


@pytest.mark.parametrize("P,N,io,L,B,H,G", [
    (16, 16, "f32", 1, 3, 6, 3),
    (16, 16, "bf16", 5, 5, 4, 2),
    (64, 64, "bf16", 3, 7, 6, 1),
    (64, 128, "f32", 7, 3, 12, 4),
    (64, 128, "bf16", 32, 2, 16, 8),
    (128, 128, "bf16", 8, 3, 5, 5),
])
def test_ragged_shapes(P, N, io, L, B, H, G):
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L,
                       io_dtype=io, config=synth.CONFIG_ID["misc"], layer=P + N + L)
    _standard_case(w, 2 * L + 3, list(range(B)))


def test_decode_workload_first_windows():
    """Mamba-2-shaped layer, full batch 256, 128 heads, 8 groups, P=64, N=128,
    L=16: the first 3 windows, 6 sampled sequences."""
    w = synth.named("decode")
    _standard_case(w, 48, [0, 1, 77, 128, 200, 255])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_dyadic_bit_exact(io):
    """Inputs whose whole recurrence is exact in float32: the GPU outputs and
    the flushed checkpoint equal the float64 oracle bit for bit."""
    w = synth.Workload(batch=4, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=8,
                       io_dtype=io, config=synth.CONFIG_ID["misc"], layer=3)
    T = 8
    gu.note(f"dyadic {io}")
    inp = synth.dyadic_inputs(w, 0, T)
    dev = {k: gu.to_dev(v) for k, v in inp.items()}
    layer = _layer(w)
    y = torch.empty((T, 4, 8, 64), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.append(1, dev["q"][t], dev["k"][t], dev["v"][t], dev["dt"][t], dev["a"][t])
        layer.decode(y[t])
        if t == 5:
            layer.flush(1)      # one flush mid-run: checkpoint path exercised too
    torch.cuda.synchronize()
    x = runs.widen_inputs(inp, io)
    S = np.zeros((4, 8, 64, 128))
    y_ref = runs.standard(x, S)
    assert np.array_equal(y_ref.astype(np.float32).astype(np.float64), y_ref), "oracle not fp32-exact"
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)
    S6 = np.zeros((4, 8, 64, 128))
    runs.standard({k: v[:6] for k, v in x.items()}, S6)
    assert np.array_equal(layer.s_master.cpu().numpy().astype(np.float64), S6)
    layer.close()
