"""replay_step_static: the decode step for callers that cannot allocate
device memory, whose arrival counters live in the library's static array
instead of the layer's `sync` buffer.  Through the C ABI, against
replay_step on the same inputs: outputs, checkpoints, copies and pointers
bit for bit, step after step (folds included), for a layer of 6 sequences
and then, on the same static array, a smaller layer of 2; a float32
checkpoint (one fused launch), an e4m3 copy (the copy-mode launch, then
the flush kernel, both on the static counters) and a Gated DeltaNet layer
(append, output-only and fold launches, the append and the fold on the
static counters).  A layer needing more
counters than the array holds is refused before any launch; a layer built
without counters refuses the calls that need them."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _layer(w, **kw):
    import linear_attention_decode_amd as lad
    return lad.ReplayLayer(w.batch, w.heads, w.groups, w.head_dim, w.state_dim, w.ring_len,
                           io_dtype=w.io_dtype, device=gu.DEV, **kw)


class _GdnInputs(gu.DevInputs):
    """Gated DeltaNet inputs (unit-length q, k; beta in the dt slot, alpha in the a slot)."""

    def __init__(self, w, t0, t1):
        self.w = w
        self.t0 = t0
        self.t = {k: gu.to_dev(v) for k, v in synth.gdn_inputs(w, t0, t1).items()}


@pytest.mark.parametrize("copy,rule", [(None, "mamba2"), ("fp8", "mamba2"), (None, "gdn")])
def test_step_static_equals_step(copy, rule):
    for B in (6, 2):                      # two layers in a row, the second smaller
        w = synth.Workload(batch=B, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=4, io_dtype="bf16",
                           config=synth.CONFIG_ID["misc"], layer=400 + B)
        T = 3 * w.ring_len + 1
        gu.note(f"step_static vs step B={B} copy={copy} rule={rule}")
        dev = _GdnInputs(w, 0, T) if rule == "gdn" else gu.DevInputs(w, 0, T)
        kw = {"rule": rule} if copy is None else {"read_copy": copy, "rule": rule}
        st = _layer(w, counters=False, **kw)
        ref = _layer(w, **kw)
        assert st.sync is None
        ys = torch.empty((B, w.heads, w.head_dim), dtype=torch.float32, device=gu.DEV)
        yr = torch.empty_like(ys)
        for t in range(T):
            st.step_static(*dev.step(t), ys, flush_at=w.ring_len)
            ref.step(*dev.step(t), yr, flush_at=w.ring_len)
            torch.cuda.synchronize()
            assert torch.equal(ys, yr), (B, t)
            assert torch.isfinite(ys).all()
            for name in ("pos", "base", "s_master", "s_copy", "s_scale"):
                if st.t[name] is not None:
                    assert torch.equal(st.t[name], ref.t[name]), (B, t, name)
        assert st.get_error()[0] == 0 and ref.get_error()[0] == 0
        assert st.base.cpu().tolist() == [3 * w.ring_len] * B
        st.close()
        ref.close()


def test_step_static_limits():
    import linear_attention_decode_amd as lad
    # 2048 sequences x 9 counters x 128 bytes > 2 MiB: refused, nothing enqueued
    w = synth.Workload(batch=2048, heads=8, groups=8, head_dim=16, state_dim=16, ring_len=2, io_dtype="f32",
                       config=synth.CONFIG_ID["misc"], layer=410)
    gu.note("step_static too large")
    big = _layer(w, counters=False)
    dev = gu.DevInputs(w, 0, 1)
    y = torch.full((w.batch, w.heads, w.head_dim), 7.0, dtype=torch.float32, device=gu.DEV)
    with pytest.raises(lad.ReplayError, match="status 4"):
        big.step_static(*dev.step(0), y)
    # the calls that need the layer's own counters refuse a layer built without them
    with pytest.raises(lad.ReplayError, match="status 1"):
        big.step(*dev.step(0), y)
    with pytest.raises(lad.ReplayError, match="status 1"):
        big.flush(1)
    torch.cuda.synchronize()
    assert big.pos.cpu().eq(0).all() and bool((y == 7.0).all())
    big.close()
