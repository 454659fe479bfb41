"""The ring's documented layouts, read back after each call that writes it.

Every kernel reads the ring through the same layout it was written with, so
parity tests alone would not notice a layout that differs from the one the
C ABI documents.  After appends (replay_append), fused steps (writer
workgroups) and fused verify rounds (drafts; register and matrix-core
windows), the ring slots must hold the inputs bit for bit where the header
says: v [B][H][L][P], q and k [B][G][L][N], dt and a [B][L][H]
(slot-major), token n of a sequence in slot n mod L -- also past the ring's
end, where the slots wrap."""
import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("route,n", [("append", 4), ("step", 5), ("verify_step", 4), ("verify_step", 6)])
def test_ring_layout(route, n):
    import linear_attention_decode_amd as lad
    L, pre = 8, 6
    w = synth.Workload(batch=3, heads=8, groups=2, head_dim=64, state_dim=128, ring_len=L, io_dtype="bf16",
                       config=synth.CONFIG_ID["misc"], layer=450)
    B, H, P, N = w.batch, w.heads, w.head_dim, w.state_dim
    gu.note(f"ring layout via {route} n={n}")
    dev = gu.DevInputs(w, 0, pre + n)
    layer = lad.ReplayLayer(B, H, w.groups, P, N, L, io_dtype="bf16", device=gu.DEV)
    layer.load_checkpoint(torch.zeros((B, H, P, N), dtype=torch.float32, device=gu.DEV))
    # tokens 0..5 fill slots 0..5 and are folded, so the route's tokens start
    # at slot 6 and wrap to slot 0
    layer.append(pre, *dev.window(0, pre))
    layer.flush(1)
    if route == "append":
        layer.append(n, *dev.window(pre, n))
    elif route == "step":
        y = torch.empty((B, H, P), dtype=torch.float32, device=gu.DEV)
        for t in range(pre, pre + n):
            layer.step(*dev.step(t), y, flush_at=L + 1)          # never folds
    else:
        y = torch.empty((B, n, H, P), dtype=torch.float32, device=gu.DEV)
        layer.verify_step(n, *dev.window(pre, n), y, flush_at=L + 1)
    torch.cuda.synchronize()
    assert layer.get_error()[0] == 0
    assert layer.pos.cpu().tolist() == [pre + n] * B and layer.base.cpu().tolist() == [pre] * B
    rv, rq, rk = layer.ring_v.cpu(), layer.ring_q.cpu(), layer.ring_k.cpu()
    rdt, ra = layer.ring_dt.cpu(), layer.ring_a.cpu()
    assert tuple(rdt.shape) == (B, L, H) and tuple(rv.shape) == (B, H, L, P)
    for t in range(pre, pre + n):
        q, k, v, dt, a = (x.cpu() for x in dev.step(t))
        s = t % L
        assert torch.equal(rv[:, :, s], v), (t, "v")
        assert torch.equal(rq[:, :, s], q), (t, "q")
        assert torch.equal(rk[:, :, s], k), (t, "k")
        assert torch.equal(rdt[:, s, :], dt), (t, "dt")
        assert torch.equal(ra[:, s, :], a), (t, "a")
    layer.close()
