"""Decode steps and verify rounds recorded into a HIP graph and replayed.

One graph holds a step (or a verify round plus its rollback) of one or
several stacked layers.  Before each replay the next inputs are copied into
the buffers the graph was captured with; an eager twin of every layer makes
the same calls with the same inputs.  After every replay, with the eager
work and a synchronisation in between, the outputs, pos, base and the error
bits must equal the twin's bit for bit, and at the end an eager flush of
both must leave identical checkpoints.  The copy-mode steps end in a flush
kernel that the handle may skip on its host-side count bounds, so a capture
taken while no sequence was due must still record it.  Gated DeltaNet
layers (their step is the append, output-only and fold launches in turn;
their rounds the flush, append and matrix-core verify) are recorded the
same way."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

L = 8


def _workload(layer, P=64, N=128):
    return synth.Workload(batch=4, heads=8, groups=2, head_dim=P, state_dim=N, ring_len=L, io_dtype="bf16",
                          config=synth.CONFIG_ID["misc"], layer=500 + layer)


def _pair(w, rc, rule="mamba2"):
    import linear_attention_decode_amd as lad
    kw = {} if rc is None else {"read_copy": rc}
    mk = lambda: lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, L, io_dtype="bf16",
                                 device=gu.DEV, rule=rule, **kw)
    return mk(), mk()


class _GdnInputs(gu.DevInputs):
    """Gated DeltaNet inputs (unit-length q, k; beta in the dt slot, alpha in the a slot)."""

    def __init__(self, w, t0, t1):
        self.w = w
        self.t0 = t0
        self.t = {k: gu.to_dev(v) for k, v in synth.gdn_inputs(w, t0, t1).items()}


def _inputs(w, t0, t1, rule):
    return _GdnInputs(w, t0, t1) if rule == "gdn" else gu.DevInputs(w, t0, t1)


def _same_state(e, g, what):
    assert torch.equal(e.pos, g.pos) and torch.equal(e.base, g.base), what
    we, pe = e.get_error()
    wg, pg = g.get_error()
    assert (we, pe) == (wg, pg), (what, pe, pg)


@pytest.mark.parametrize("rc,layers,P,N,rule", [(None, 1, 64, 128, "mamba2"), ("fp8", 1, 64, 128, "mamba2"),
                                                ("bf16", 1, 64, 128, "mamba2"), (None, 3, 64, 128, "mamba2"),
                                                (None, 2, 128, 128, "mamba2"), ("fp8", 1, 128, 128, "mamba2"),
                                                (None, 2, 128, 128, "gdn"), ("fp4", 1, 64, 128, "gdn")])
def test_graph_steps(rc, layers, P, N, rule):
    """128 x 128 heads: two workgroups per head in the single-launch step."""
    gu.note(f"graph of steps copy={rc} layers={layers} P={P} N={N} rule={rule}")
    T0, T = 2, 3 * L + 3
    ws = [_workload(i, P, N) for i in range(layers)]
    devs = [_inputs(w, 0, T, rule) for w in ws]
    pairs = [_pair(w, rc, rule) for w in ws]
    B, H, P = ws[0].batch, ws[0].heads, ws[0].head_dim
    ys = [(torch.empty((B, H, P), dtype=torch.float32, device=gu.DEV),
           torch.empty((B, H, P), dtype=torch.float32, device=gu.DEV)) for _ in ws]
    for t in range(T0):   # eager on both (count T0 at capture: no sequence due)
        for (e, g), d, (ye, yg) in zip(pairs, devs, ys):
            e.step(*d.step(t), ye, flush_at=L)
            g.step(*d.step(t), yg, flush_at=L)
    static = [tuple(x.clone() for x in d.step(T0)) for d in devs]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (_, g), st, (_, yg) in zip(pairs, static, ys):
            g.step(*st, yg, flush_at=L)
    for t in range(T0, T):
        for st, d in zip(static, devs):
            for dst, src in zip(st, d.step(t)):
                dst.copy_(src)
        graph.replay()
        for (e, _), d, (ye, _) in zip(pairs, devs, ys):
            e.step(*d.step(t), ye, flush_at=L)
        torch.cuda.synchronize()
        for i, ((e, g), (ye, yg)) in enumerate(zip(pairs, ys)):
            assert torch.equal(ye, yg), (t, i)
            _same_state(e, g, (t, i))
    assert int(pairs[0][0].base[0]) >= 2 * L          # the window folded on replays
    for e, g in pairs:
        e.flush(1)
        g.flush(1)    # eager, after replays the handle did not see
        torch.cuda.synchronize()
        _same_state(e, g, "final flush")
        assert int(g.base[0]) == T
        for name in ("s_master", "s_copy", "s_scale"):
            if e.t[name] is not None:
                assert torch.equal(e.t[name], g.t[name]), name
    del graph
    for e, g in pairs:
        e.close()
        g.close()


@pytest.mark.parametrize("rc,W,rule", [(None, 4, "mamba2"), (None, 6, "mamba2"), ("fp8", 4, "mamba2"),
                                       (None, 4, "gdn"), ("fp8", 5, "gdn")])
def test_graph_verify_rounds(rc, W, rule):
    """A verify round + rollback in one graph; accepted counts change per
    replay.  W = 4 and 6: the single-launch round (register sums, matrix
    cores); an e4m3 copy: flush, append and verify in turn, where the flush
    is one the bounds would skip at capture."""
    R = 12
    gu.note(f"graph of verify rounds copy={rc} W={W} rule={rule}")
    w = _workload(7)
    B, H, P = w.batch, w.heads, w.head_dim
    dev = _inputs(w, 0, (R + 1) * W, rule)
    e, g = _pair(w, rc, rule)
    accept = np.random.default_rng(3).integers(0, W + 1, size=(R + 1, B))
    nrej = [torch.from_numpy((W - a).astype(np.int32)).to(gu.DEV) for a in accept]
    ye = torch.empty((B, W, H, P), dtype=torch.float32, device=gu.DEV)
    yg = torch.empty_like(ye)
    fa = L - W + 1
    for x in (e, g):   # one eager round on both
        x.verify_step(W, *dev.window(0, W), ye if x is e else yg, flush_at=fa)
        x.rollback(nrej[0])
    static = tuple(x.clone() for x in dev.window(W, W))
    s_rej = nrej[1].clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.verify_step(W, *static, yg, flush_at=fa)
        g.rollback(s_rej)
    folds = 0
    for r in range(1, R + 1):
        for dst, src in zip(static, dev.window(r * W, W)):
            dst.copy_(src)
        s_rej.copy_(nrej[r])
        base0 = g.base.clone()
        graph.replay()
        e.verify_step(W, *dev.window(r * W, W), ye, flush_at=fa)
        e.rollback(nrej[r])
        torch.cuda.synchronize()
        assert torch.equal(ye, yg), r
        _same_state(e, g, r)
        folds += int((g.base != base0).sum())
    assert folds > 0
    e.flush(1)
    g.flush(1)
    torch.cuda.synchronize()
    _same_state(e, g, "final flush")
    for name in ("s_master", "s_copy", "s_scale"):
        if e.t[name] is not None:
            assert torch.equal(e.t[name], g.t[name]), name
    del graph
    e.close()
    g.close()


@pytest.mark.parametrize("rc,W", [(None, 4), (None, 6), ("fp8", 4)])
def test_graph_rollback_verify_rounds(rc, W):
    """replay_rollback_verify_step in a graph: each replay rolls back the
    previous round (the reject counts change per replay) and runs the next
    round in one launch (register sums at W = 4, matrix cores at W = 6, an
    e4m3 copy's round); an eager twin runs replay_rollback then
    replay_verify_step.  Outputs, pointers and error bits equal after every
    replay, checkpoints after a final flush."""
    R = 10
    gu.note(f"graph of rollback + verify rounds copy={rc} W={W}")
    w = _workload(9)
    B, H, P = w.batch, w.heads, w.head_dim
    dev = _inputs(w, 0, (R + 1) * W, "mamba2")
    e, g = _pair(w, rc, "mamba2")
    accept = np.random.default_rng(5).integers(0, W + 1, size=(R + 1, B))
    nrej = [torch.from_numpy((W - a).astype(np.int32)).to(gu.DEV) for a in accept]
    ye = torch.empty((B, W, H, P), dtype=torch.float32, device=gu.DEV)
    yg = torch.empty_like(ye)
    fa = L - W + 1
    for x in (e, g):   # one eager round on both; its rollback is pending
        x.verify_step(W, *dev.window(0, W), ye if x is e else yg, flush_at=fa)
    static = tuple(x.clone() for x in dev.window(W, W))
    s_rej = nrej[0].clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.rollback_verify_step(s_rej, W, *static, yg, flush_at=fa)
    for r in range(1, R + 1):
        for dst, src in zip(static, dev.window(r * W, W)):
            dst.copy_(src)
        s_rej.copy_(nrej[r - 1])
        graph.replay()
        e.rollback(nrej[r - 1])
        e.verify_step(W, *dev.window(r * W, W), ye, flush_at=fa)
        torch.cuda.synchronize()
        assert torch.equal(ye, yg), r
        _same_state(e, g, r)
    for x in (e, g):
        x.rollback(nrej[R])
        x.flush(1)
    torch.cuda.synchronize()
    _same_state(e, g, "final flush")
    for name in ("s_master", "s_copy", "s_scale"):
        if e.t[name] is not None:
            assert torch.equal(e.t[name], g.t[name]), name
    del graph
    e.close()
    g.close()
