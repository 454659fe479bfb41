"""replay_step_layers: the fused decode step of several stacked layers of
one shape in a single launch.

- Against replay_step on each layer in turn: outputs after every step,
  checkpoints, pointers and ring slots bit for bit (the same kernel code),
  over ragged shapes, both ring bounds, folds every L steps and two
  workgroups per 128 x 128 head.
- The stacked workload's shapes (8 layers, B=512, H=64, G=8, P=N=128,
  L=16), 32 steps (2 folds; a layer of this size is stepped one launch
  each), and the same layers at B=32 (one launch for all): sampled
  sequences of every layer against the float64 oracle (1e-4 per head,
  floored as tests/parity.py states), and every layer's outputs equal to
  replay_step's bit for bit.
- The call recorded into a HIP graph and replayed equals eager calls.
- Host-side errors: layer counts outside 1..16, mismatched shapes, the same
  layer twice, a copy-mode layer."""
import numpy as np
import pytest
import torch

import synth
from oracle import runs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
RING = ("ring_q", "ring_k", "ring_v", "ring_dt", "ring_a")


def _lad():
    import linear_attention_decode_amd as lad
    return lad


def _layer(w, **kw):
    layer = _lad().ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                               io_dtype=w.io_dtype, device=gu.DEV, **kw)
    for name in RING:
        layer.t[name].zero_()
    return layer


def _step_all(layers, ins, ys, flush_at):
    """ins: per layer (q, k, v, dt, a) tuples; ys: per layer outputs."""
    cols = list(zip(*ins))
    _lad().replay_step_layers([l.h for l in layers], *cols, ys, flush_at)


@pytest.mark.parametrize("P,N,io,L,flush_at,B,H,G,n", [
    (64, 128, "bf16", 16, 16, 3, 8, 2, 3),
    (128, 128, "bf16", 8, 8, 2, 4, 2, 5),      # two workgroups per head
    (16, 16, "f32", 4, 4, 3, 6, 3, 2),
    (64, 64, "bf16", 32, 32, 2, 4, 1, 4),      # two ring wavefronts per head
    (64, 128, "f32", 7, 3, 2, 8, 4, 2),
    (64, 128, "bf16", 6, 1, 3, 8, 8, 16),      # the most layers one launch takes; fold every step
])
def test_layers_equal_steps(P, N, io, L, flush_at, B, H, G, n):
    ws = [synth.Workload(batch=B, heads=H, groups=G, head_dim=P, state_dim=N, ring_len=L, io_dtype=io,
                         config=synth.CONFIG_ID["misc"], layer=600 + 10 * i + L) for i in range(n)]
    T = 2 * L + 3
    gu.note(f"step_layers vs steps n={n} {ws[0]} flush_at={flush_at}")
    devs = [gu.DevInputs(w, 0, T) for w in ws]
    one = [_layer(w) for w in ws]
    each = [_layer(w) for w in ws]
    y1 = [torch.empty((B, H, P), dtype=torch.float32, device=gu.DEV) for _ in ws]
    ye = [torch.empty_like(y) for y in y1]
    for t in range(T):
        _step_all(one, [d.step(t) for d in devs], y1, flush_at)
        for lay, d, y in zip(each, devs, ye):
            lay.step(*d.step(t), y, flush_at=flush_at)
        torch.cuda.synchronize()
        for i in range(n):
            assert torch.equal(y1[i], ye[i]), (t, i)
            assert torch.isfinite(y1[i]).all()
    for i in range(n):
        assert one[i].get_error()[0] == 0 and each[i].get_error()[0] == 0
        for name in ("s_master", "pos", "base") + RING:
            assert torch.equal(one[i].t[name], each[i].t[name]), (i, name)
        assert torch.equal(one[i].sync, torch.zeros_like(one[i].sync))
        one[i].close()
        each[i].close()


@pytest.mark.parametrize("B", [512, 32])
def test_layers_stacked_workload(B):
    T, L = 32, 16
    seqs = [0, B // 2 - 1, B - 1]
    ws = [synth.named("stacked", ring_len=L, layer=li, batch=B) for li in range(8)]
    gu.note(f"step_layers stacked workload {ws[0]} T={T}")
    devs = [gu.DevInputsTorch(w, 0, T) for w in ws]
    one = [_layer(w) for w in ws]
    B, H, P = ws[0].batch, ws[0].heads, ws[0].head_dim
    ys = [torch.empty((T, B, H, P), dtype=torch.float32, device=gu.DEV) for _ in ws]
    for t in range(T):
        _step_all(one, [d.step(t) for d in devs], [y[t] for y in ys], L)
    torch.cuda.synchronize()
    for li, (w, d) in enumerate(zip(ws, devs)):
        assert one[li].get_error()[0] == 0
        assert one[li].base.cpu().tolist() == [T] * B
        x = d.oracle(seqs)
        y_ref = runs.standard(x, np.zeros((len(seqs), H, P, w.state_dim)))
        y_abs = gu.y_abs_standard(x, (len(seqs), H, P, w.state_dim))
        gu.assert_f32(ys[li].cpu().numpy()[:, seqs], y_ref, y_abs, what=f"layer {li}:")
    # every layer, every sequence: the same bits as replay_step on that layer alone
    for li, (w, d) in enumerate(zip(ws, devs)):
        lay = _layer(w)
        y = torch.empty((B, H, P), dtype=torch.float32, device=gu.DEV)
        for t in range(T):
            lay.step(*d.step(t), y, flush_at=L)
            assert torch.equal(y, ys[li][t]), (li, t)
        torch.cuda.synchronize()
        assert torch.equal(lay.s_master, one[li].s_master), li
        lay.close()
        one[li].close()


def test_layers_graph_replay():
    n, L = 3, 8
    ws = [synth.Workload(batch=4, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=L, io_dtype="bf16",
                         config=synth.CONFIG_ID["misc"], layer=650 + i) for i in range(n)]
    T0, T = 2, 3 * L + 3
    gu.note("step_layers graph replay")
    devs = [gu.DevInputs(w, 0, T) for w in ws]
    eager = [_layer(w) for w in ws]
    graphed = [_layer(w) for w in ws]
    ye = [torch.empty((4, 8, 64), dtype=torch.float32, device=gu.DEV) for _ in ws]
    yg = [torch.empty_like(y) for y in ye]
    for t in range(T0):
        _step_all(eager, [d.step(t) for d in devs], ye, L)
        _step_all(graphed, [d.step(t) for d in devs], yg, L)
    static = [tuple(x.clone() for x in d.step(T0)) for d in devs]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step_all(graphed, static, yg, L)
    for t in range(T0, T):
        for st, d in zip(static, devs):
            for dst, src in zip(st, d.step(t)):
                dst.copy_(src)
        graph.replay()
        _step_all(eager, [d.step(t) for d in devs], ye, L)
        torch.cuda.synchronize()
        for i in range(n):
            assert torch.equal(ye[i], yg[i]), (t, i)
            assert torch.equal(eager[i].pos, graphed[i].pos) and torch.equal(eager[i].base, graphed[i].base)
    assert int(graphed[0].base[0]) >= 2 * L
    for e, g in zip(eager, graphed):
        e.flush(1)
        g.flush(1)
        torch.cuda.synchronize()
        assert torch.equal(e.s_master, g.s_master)
        assert e.get_error()[0] == 0 and g.get_error()[0] == 0
        e.close()
        g.close()


def test_layers_errors():
    lad = _lad()
    mk = lambda layer, **kw: synth.Workload(batch=2, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=4,
                                            io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=layer, **kw)
    gu.note("step_layers errors")
    w = mk(660)
    d = gu.DevInputs(w, 0, 1)
    a, b = _layer(w), _layer(w)
    other = _layer(synth.Workload(batch=3, heads=4, groups=2, head_dim=64, state_dim=128, ring_len=4,
                                  io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=661))
    cp = _layer(w, read_copy="fp8")
    y = torch.full((2, 4, 64), 5.0, dtype=torch.float32, device=gu.DEV)
    ins = d.step(0)
    cases = [([a, b, other], 1), ([a, a], 1), ([a, cp], 2), ([a] * 17, 1)]
    for layers, status in cases:
        with pytest.raises(lad.ReplayError, match=f"status {status}"):
            _step_all(layers, [ins] * len(layers), [y] * len(layers), 4)
    with pytest.raises(lad.ReplayError, match="status 1"):
        lad.replay_step_layers([], [], [], [], [], [], [], 4)
    torch.cuda.synchronize()
    assert bool((y == 5.0).all()) and a.pos.cpu().eq(0).all() and b.pos.cpu().eq(0).all()
    for lay in (a, b, other, cp):
        lay.close()
