"""MX FP4 read copy on the GPU: separated precisions (the float32 master
takes every flush, outputs read the FP4 copy) and shared (the FP4 copy is
the only checkpoint: every flush dequantises it, folds and rewrites it).

* storage: the codes and E8M0 block scales the flush writes from a float32
  checkpoint equal the oracle's MX quantiser bit for bit (zero blocks,
  exactly representable blocks, ties and tiny blocks included);
* outputs against the oracle's emulation of the same copy (the two differ
  only where the float32 master and the float64 state round a value to
  different sides of a code boundary), and against the exact oracle within
  the format's own error as the emulation realises it (plus that slack).

No FP4 tolerance is stated; the bound used is the emulation's own
error: FP4 keeps 2 significant bits, so the copy's error is a property of
the format, and the kernels must add nothing beyond float32 rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL_VS_EMUL = gu.COPY_TOL_MAX["fp4"]


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    return lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                           io_dtype=w.io_dtype, device=gu.DEV, **kw)


def _crafted(w):
    S = synth.checkpoint_state(w, scale=0.7)
    S[0, 0] = 0.0                                             # all-zero blocks
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, S[0, 1].size).astype(np.uint8)
    S[0, 1] = (oracle.core.e2m1_decode(codes) * np.float32(2.0 ** -3)).reshape(S[0, 1].shape)   # exact values
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=np.float32)
    S[0, 2] = np.resize(np.concatenate([ties, -ties]), S[0, 2].size).reshape(S[0, 2].shape)     # ties (X = 1)
    S[1, 0] *= np.float32(1e-36)                               # tiny blocks (scale near the bottom)
    S[1, 1, :, :] *= np.float32(3e4)
    return S


@pytest.mark.parametrize("P,N,shared", [(64, 128, False), (16, 16, False), (128, 128, False), (64, 128, True),
                                        (16, 16, True)])
def test_fp4_codes_bit_exact(P, N, shared):
    w = synth.Workload(batch=3, heads=4, groups=2, head_dim=P, state_dim=N, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=70 + P)
    gu.note(f"fp4 codes P={P} N={N} shared={shared}")
    S = _crafted(w)
    layer = _layer(w, read_copy="fp4", shared_lowp=shared)
    layer.load_checkpoint(gu.to_dev(S))
    torch.cuda.synchronize()
    packed, scale = oracle.core.quant_blocks_mxfp4(S)
    got_c = layer.s_copy.cpu().numpy().reshape(packed.shape)
    got_s = layer.s_scale.cpu().numpy().reshape(scale.shape)
    assert np.array_equal(got_s, scale), np.argwhere(got_s != scale)[:5]
    mism = np.argwhere(got_c != packed)
    assert mism.size == 0, (mism[:5], got_c[tuple(mism[0])], packed[tuple(mism[0])])
    if not shared:
        assert np.array_equal(layer.s_master.cpu().numpy(), S)
    assert layer.base.cpu().tolist() == layer.pos.cpu().tolist()
    layer.close()


def _check(y_gpu, x, S0, L, label, shared=False):
    y_exact = runs.standard(x, S0.copy())
    y_emul = (runs.shared if shared else runs.separated)(x, S0.copy(), L, "fp4")
    tok_e, vec_e, _ = gu.errors(y_gpu, y_emul)
    e_gpu = runs.normwise_rel_err(y_gpu, y_exact)
    e_emul = runs.normwise_rel_err(y_emul.astype(np.float64), y_exact)
    print(f"  {label}: vs emulation per-token max {tok_e:.3e}; vs exact max {e_gpu.max():.3e} "
          f"(the emulation's own {e_emul.max():.3e})")
    gu.assert_copy(y_gpu, y_emul, "fp4", label)
    assert np.all(e_gpu <= 1.1 * e_emul + TOL_VS_EMUL)


@pytest.mark.parametrize("shared", [False, True])
def test_fp4_dual_precision_workload(shared):
    """Dual-precision shapes (B=256, H=128, G=8, P=64, N=128, L=16), full
    batch, 64 steps through replay_step, 4 sampled sequences; separated (the
    float32 master takes the folds) and shared (each fold starts from the FP4
    copy and rewrites it)."""
    w = synth.named("dual")
    T, seqs = 64, [0, 97, 160, 255]
    gu.note(f"fp4 dual precision workload shared={shared}")
    dev = synth.step_inputs_torch(w, 0, T, device=gu.DEV)
    layer = _layer(w, read_copy="fp4", shared_lowp=shared)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["dt"][t], dev["a"][t], y[t], flush_at=w.ring_len)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = runs.widen_inputs({k: synth.to_storage(v[:, seqs]) for k, v in dev.items()}, w.io_dtype)
    _check(y.cpu().numpy()[:, seqs], x, np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim)), w.ring_len,
           "dual workload", shared)
    layer.close()


@pytest.mark.parametrize("P,N,io,L,B,H,G,shared", [
    (16, 16, "f32", 4, 3, 6, 3, False),
    (64, 64, "bf16", 5, 5, 4, 2, False),
    (128, 128, "bf16", 8, 3, 4, 2, False),
    (64, 128, "f32", 32, 2, 8, 4, False),
    (16, 16, "f32", 4, 3, 6, 3, True),
    (64, 64, "bf16", 5, 5, 4, 2, True),
    (128, 128, "bf16", 8, 3, 4, 2, True),
])
def test_fp4_ragged(P, N, io, L, B, H, G, shared):
    """Decode through append / decode / flush with the FP4 copy, ragged shapes,
    starting from a non-zero checkpoint (so the copy matters from step 0);
    separated, and shared (each flush starts from the FP4 copy)."""
    w = synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=300 + P + L)
    T = 3 * L + 2
    gu.note(f"fp4 ragged {w} shared={shared}")
    S0 = synth.checkpoint_state(w, scale=0.5)
    dev = gu.DevInputs(w, 0, T)
    layer = _layer(w, read_copy="fp4", shared_lowp=shared)
    layer.load_checkpoint(gu.to_dev(S0))
    y = torch.empty((T, B, H, P), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.append(1, *dev.step(t))
        layer.decode(y[t])
        layer.flush(L)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, T, list(range(B)))
    _check(y.cpu().numpy(), x, S0.astype(np.float64), L, f"P={P} N={N} L={L}", shared)
    layer.close()


def test_fp4_verify_rounds():
    """Speculative rounds (W = 5) reading the FP4 copy: every window position
    against the oracle's emulation of the copy under the same schedule."""
    w = synth.Workload(batch=4, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=16, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=330)
    R, W = 12, 5
    gu.note("fp4 verify rounds")
    accept = synth.accept_counts(w, R, W)
    dev = gu.DevInputs(w, 0, R * W)
    layer = _layer(w, read_copy="fp4")
    y = gu.run_verify(layer, w, dev, R, W, accept)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, R * W, list(range(w.batch)))
    S0 = np.zeros((w.batch, w.heads, w.head_dim, w.state_dim))
    y_emul = runs.verify_rounds_copy(x, accept, W, S0, w.ring_len, "fp4")      # [R][W][B][H][P]
    y_exact = runs.verify_rounds(x, accept, W, S0.copy())
    y_gpu = y.cpu().numpy().transpose(0, 2, 1, 3, 4)                             # -> [R][W][B][H][P]
    tok_e, _, _ = gu.errors(y_gpu, y_emul)
    e_gpu = runs.normwise_rel_err(y_gpu, y_exact)
    e_emul = runs.normwise_rel_err(y_emul, y_exact)
    print(f"  verify: vs emulation per-token max {tok_e:.3e}; vs exact max {e_gpu.max():.3e} "
          f"(the emulation's own {e_emul.max():.3e})")
    gu.assert_copy(y_gpu, y_emul, "fp4", "verify")
    assert np.all(e_gpu <= 1.1 * e_emul + TOL_VS_EMUL)
    layer.close()
