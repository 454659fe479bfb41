"""Dual-precision checkpoints on the GPU.

* storage codes: the bf16 / e4m3 copy the library writes from a float32
  checkpoint equals the oracle's quantisers bit for bit (codes and per-head
  scales), ties and zero heads included;
* outputs read from the copies, separated (float32 master takes the
  updates) and shared (the copy is the only checkpoint), against
  - the float64 oracle with the stated tolerances (2e-2 bf16, 6e-2 e4m3,
    read per token over the layer output), and
  - the oracle's emulation of the same copy (it differs from the GPU only by
    float32-vs-float64 rounding of the state that is copied: tests/gpu_util.py
    assert_copy bounds the maximum and the median).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL_VS_EXACT = {"bf16": 2e-2, "fp8": 6e-2}


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    return lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                           io_dtype=w.io_dtype, device=gu.DEV, **kw)


def _crafted_checkpoint(w):
    S = synth.checkpoint_state(w, scale=0.7)
    # a zero head, a head with amax 448 whose entries sit exactly on e4m3 ties
    # (scale 1), and a head of exact bf16 ties (low 16 bits 0x8000)
    S[0, 0] = 0.0
    ties = np.array([1.0625, 1.1875, 3 * 2.0 ** -10, -2.5625, 13.0, 448.0], dtype=np.float32)
    S[0, 1] = np.resize(ties, S[0, 1].shape)
    bits = (np.arange(S[0, 2].size, dtype=np.uint32) % 512 + 0x3F80) << 16 | 0x8000
    S[0, 2] = bits.view(np.float32).reshape(S[0, 2].shape)
    return S


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("shared", [False, True])
def test_copy_codes_bit_exact(fmt, shared):
    w = synth.Workload(batch=3, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=61)
    gu.note(f"copy codes {fmt} shared={shared}")
    S = _crafted_checkpoint(w)
    layer = _layer(w, read_copy=fmt, shared_lowp=shared)
    layer.load_checkpoint(gu.to_dev(S))
    torch.cuda.synchronize()
    if fmt == "bf16":
        got = layer.s_copy.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, oracle.bf16_encode(S))
    else:
        codes, scale = oracle.quant_heads_e4m3(S)
        got = layer.s_copy.cpu().numpy()
        assert np.array_equal(layer.s_scale.cpu().numpy(), scale)
        mism = np.argwhere(got != codes)
        assert mism.size == 0, (mism[:5], got[tuple(mism[0])], codes[tuple(mism[0])])
    if not shared:
        assert np.array_equal(layer.s_master.cpu().numpy(), S)
    assert layer.base.cpu().tolist() == layer.pos.cpu().tolist()
    layer.close()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("route", ["step", "verify_step"])
def test_copy_codes_after_folds_bit_exact(fmt, route):
    """Separated precisions: after folds (fused steps with the flush, or
    fused speculative rounds), the copy's codes and scales equal the
    oracle's quantisers applied to the float32 master the same launch wrote,
    bit for bit (the e4m3 division by the head's scale included)."""
    w = synth.Workload(batch=4, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=8,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=62)
    gu.note(f"copy codes after folds {fmt} {route}")
    layer = _layer(w, read_copy=fmt)
    layer.load_checkpoint(gu.to_dev(synth.checkpoint_state(w, scale=0.6)))
    if route == "step":
        T = 27
        dev = gu.DevInputs(w, 0, T)
        y = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
        for t in range(T):
            layer.step(*dev.step(t), y, flush_at=w.ring_len)
    else:
        R, W = 9, 4
        gu.run_verify(layer, w, gu.DevInputs(w, 0, R * W), R, W, synth.accept_counts(w, R, W), fused=True)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    assert (layer.base.cpu() > 0).all()          # every sequence folded at least once
    S = layer.s_master.cpu().numpy()
    if fmt == "bf16":
        got = layer.s_copy.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, oracle.bf16_encode(S))
    elif fmt == "fp8":
        codes, scale = oracle.quant_heads_e4m3(S)
        assert np.array_equal(layer.s_scale.cpu().numpy(), scale)
        got = layer.s_copy.cpu().numpy()
        mism = np.argwhere(got != codes)
        assert mism.size == 0, (mism[:5], got[tuple(mism[0])], codes[tuple(mism[0])])
    else:
        packed, scale = oracle.core.quant_blocks_mxfp4(S)
        assert np.array_equal(layer.s_scale.cpu().numpy().reshape(scale.shape), scale)
        assert np.array_equal(layer.s_copy.cpu().numpy().reshape(packed.shape), packed)
    layer.close()


MODES = [("bf16", False), ("fp8", False), ("bf16", True), ("fp8", True)]


@pytest.mark.parametrize("fmt,shared", MODES, ids=[f"{f}-{'shared' if s else 'separated'}" for f, s in MODES])
def test_dual_precision_workload(fmt, shared):
    """Dual-precision workload shapes (B=256, H=128, G=8, P=64, N=128, L=16),
    full batch, 64 steps (4 flushes) through replay_step as the benchmark
    runs it, 4 sampled sequences."""
    w = synth.named("dual")
    T, seqs = 64, [0, 97, 160, 255]
    gu.note(f"dual precision {fmt} shared={shared}")
    dev = synth.step_inputs_torch(w, 0, T, device=gu.DEV)
    layer = _layer(w, read_copy=fmt, shared_lowp=shared)
    y = torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.step(dev["q"][t], dev["k"][t], dev["v"][t], dev["dt"][t], dev["a"][t], y[t], flush_at=w.ring_len)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = runs.widen_inputs({k: synth.to_storage(v[:, seqs]) for k, v in dev.items()}, w.io_dtype)
    y_gpu = y.cpu().numpy()[:, seqs]
    S0 = np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim))
    y_exact = runs.standard(x, S0.copy())
    y_emul = (runs.shared if shared else runs.separated)(x, S0.copy(), w.ring_len, fmt)
    tok, vec, mean = gu.errors(y_gpu, y_exact)
    tok_e, vec_e, _ = gu.errors(y_gpu, y_emul)
    print(f"  vs exact: per-token max {tok:.3e} per-head max {vec:.3e} mean {mean:.3e}; "
          f"vs emulation: per-token max {tok_e:.3e} per-head max {vec_e:.3e}")
    # the stated bound, unless the format's own error (its emulation) passes it too
    tok_fmt = gu.errors(y_emul, y_exact)[0]
    assert tok <= TOL_VS_EXACT[fmt] or tok_fmt > 0.9 * TOL_VS_EXACT[fmt]
    gu.assert_copy(y_gpu, y_emul, fmt)
    layer.close()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("P,N,H,G,L,io", [(64, 64, 4, 2, 5, "bf16"), (64, 64, 8, 2, 5, "f32"),
                                          (128, 128, 4, 2, 8, "bf16"), (16, 16, 6, 3, 4, "bf16")])
def test_shared_ragged(fmt, P, N, H, G, L, io):
    """Shared checkpoint (the copy is the only state), ragged shapes with a
    non-zero start: append / decode / flush(L) for 3L+2 steps against the
    oracle's shared emulation.  Two heads of a group fold in one workgroup
    here (H/G = 2 or 4), each wavefront staging its rows through its own LDS
    buffer; a read-back that ran ahead of another lane's writes left old
    codes in the copy after the first fold."""
    w = synth.Workload(batch=5, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                       config=synth.CONFIG_ID["misc"], layer=300 + P + L)
    T = 3 * L + 2
    gu.note(f"shared ragged {fmt} {w}")
    S0 = synth.checkpoint_state(w, scale=0.5)
    dev = gu.DevInputs(w, 0, T)
    layer = _layer(w, read_copy=fmt, shared_lowp=True)
    layer.load_checkpoint(gu.to_dev(S0))
    y = torch.empty((T, w.batch, H, P), dtype=torch.float32, device=gu.DEV)
    for t in range(T):
        layer.append(1, *dev.step(t))
        layer.decode(y[t])
        layer.flush(L)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    x = gu.oracle_inputs(w, 0, T, list(range(w.batch)))
    y_emul = runs.shared(x, S0.astype(np.float64).copy(), L, fmt)
    gu.assert_copy(y.cpu().numpy(), y_emul, fmt, f"shared {fmt} P={P} N={N}")
    layer.close()


def _drift(y_gpu, y_ref, L):
    e = runs.normwise_rel_err(y_gpu, y_ref)                # [T][b]
    nw = e.shape[0] // L
    win = e[: nw * L].reshape(nw, L, -1)
    return e, [(i, float(win[i].max()), float(win[i].mean())) for i in sorted({0, nw // 2, nw - 1})]


@pytest.mark.parametrize("dt_scale", [1.0, 0.01])
def test_dual_precision_drift(dt_scale):
    """Error drift over 1024 steps (64 windows) at the dual-precision shapes,
    full batch, 8 sequences spread over it against the float64 oracle, per
    window (first, middle, last), for the bf16, e4m3 and FP4 copies separated
    and shared.  Every mode is also run through the oracle's emulation of
    that copy (runs.separated / runs.shared): the device's error matches the
    format's own error token by token (within 1.1x plus the copy tolerance),
    and separated copies meet the stated tolerances (2e-2 bf16, 6e-2 e4m3)
    on every token where the format itself does -- the e4m3 copy's own
    error passes 6e-2 on a few tokens of the standard recipe.  With slow decay (dt x 0.01, a ~ 0.99, so the checkpoint
    carries the history) the shared low-precision checkpoint, which starts
    every flush from its own rounded copy, drifts further than the
    separated one; that comparison is what the dual-precision design is for
    ([Abstract]; [Video] takeaways), so it is asserted on mean error."""
    w = synth.named("dual", dt_scale=dt_scale)
    T, seqs, L = 1024, list(range(3, w.batch, 32)), w.ring_len
    gu.note(f"dual precision drift dt_scale={dt_scale}")
    chunks = [synth.step_inputs_torch(w, t0, t0 + 128, device=gu.DEV) for t0 in range(0, T, 128)]
    sel = torch.tensor(seqs, device=gu.DEV)
    x = runs.widen_inputs({k: np.concatenate([synth.to_storage(c[k][:, seqs]) for c in chunks])
                           for k in chunks[0]}, w.io_dtype)
    y_ref = runs.standard(x, np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim)))
    means = {}
    for fmt, shared in [("bf16", False), ("bf16", True), ("fp8", False), ("fp8", True), ("fp4", False), ("fp4", True)]:
        layer = _layer(w, read_copy=fmt, shared_lowp=shared)
        y = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
        ys = torch.empty((T, len(seqs), w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
        for t in range(T):
            c = chunks[t // 128]
            i = t % 128
            layer.step(c["q"][i], c["k"][i], c["v"][i], c["dt"][i], c["a"][i], y, flush_at=L)
            ys[t] = y.index_select(0, sel)
        torch.cuda.synchronize()
        assert layer.get_error()[0] == 0
        layer.close()
        e, win = _drift(ys.cpu().numpy(), y_ref, L)
        # the copy's own error: the oracle's emulation of the same mode
        y_em = (runs.shared if shared else runs.separated)(
            x, np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim)), L, fmt)
        e_em, win_em = _drift(y_em, y_ref, L)
        means[(fmt, shared)] = float(e.mean())
        tol = TOL_VS_EXACT.get(fmt)
        over = "" if tol is None else f"; tokens above {tol:.0e}: {int((e > tol).sum())} (emulation {int((e_em > tol).sum())}) of {e.size}"
        print(f"  {fmt} {'shared' if shared else 'separated'}: max {e.max():.3e} mean {e.mean():.3e} "
              f"(emulation max {e_em.max():.3e} mean {e_em.mean():.3e}){over}; "
              + ", ".join(f"window {i}: max {mx:.3e} mean {mn:.3e}" for i, mx, mn in win))
        # the kernels add nothing to the format's own error, token by token
        assert np.all(e <= 1.1 * e_em + gu.COPY_TOL_MAX[fmt])
        if not shared and tol is not None:
            # the stated tolerance, wherever the format itself meets it
            assert float(e.max()) <= tol or float(e_em.max()) > tol
            assert np.all((e <= tol) | (e_em > 0.9 * tol))
        if fmt == "fp4" and not shared:
            # separated: the error does not compound -- the last window's mean is no worse than the
            # middle one's (window maxima are single tokens, which a sample of 8 sequences makes noisy)
            assert win[-1][2] <= 1.2 * win[1][2] + 1e-6
    if dt_scale < 1.0:
        assert means[("fp8", True)] > 1.2 * means[("fp8", False)]
        assert means[("fp4", True)] > 1.2 * means[("fp4", False)]


@pytest.mark.parametrize("L", [8, 16, 32])
def test_stacked_layers(L):
    """Stacked sweep shapes: 8 SSM layers, B=512, H=64, G=8, P=N=128, ring
    L; 64 steps, each layer its own seeded inputs; layers 0-3 through the
    fused replay_step (the benchmark's route), 4-7 through append, decode and
    flush; 3 sampled sequences per layer against the oracle."""
    T, seqs = 64, [0, 300, 511]
    layers, ys, devs = [], [], []
    for li in range(8):
        w = synth.named("stacked", ring_len=L, layer=li)
        gu.note(f"stacked layer {li} L={L}")
        devs.append(synth.step_inputs_torch(w, 0, T, device=gu.DEV))
        layers.append(_layer(w))
        ys.append(torch.empty((T, w.batch, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV))
    for t in range(T):
        for li in range(8):
            d = devs[li]
            if li < 4:
                layers[li].step(d["q"][t], d["k"][t], d["v"][t], d["dt"][t], d["a"][t], ys[li][t], flush_at=L)
            else:
                layers[li].append(1, d["q"][t], d["k"][t], d["v"][t], d["dt"][t], d["a"][t])
                layers[li].decode(ys[li][t])
                layers[li].flush(L)
    torch.cuda.synchronize()
    for li in range(8):
        w = synth.named("stacked", ring_len=L, layer=li)
        assert layers[li].get_error()[0] == 0
        x = runs.widen_inputs({k: synth.to_storage(v[:, seqs]) for k, v in devs[li].items()}, w.io_dtype)
        y_ref = runs.standard(x, np.zeros((len(seqs), w.heads, w.head_dim, w.state_dim)))
        y_abs = gu.y_abs_standard(x, (len(seqs), w.heads, w.head_dim, w.state_dim))
        gu.assert_f32(ys[li].cpu().numpy()[:, seqs], y_ref, y_abs, what=f"layer {li}:")
        layers[li].close()
