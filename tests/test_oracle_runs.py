"""The oracle's call schedules against their limits (no GPU).

* verify rounds that accept every draft equal standard decode over the same
  tokens; rounds that accept none leave the state alone; the state after any
  accept pattern equals standard decode over the accepted prefixes only
  (rollback = recomputation from the accepted prefix).
* the dual-precision emulations: a copy format that rounds nothing
  reproduces standard decode; shared and separated agree while no flush has
  happened; separated bf16 / fp8 stay within the format's rounding of the
  exact outputs.
"""
import numpy as np

import synth
from oracle import runs

W_TINY = synth.Workload(batch=3, heads=4, groups=2, head_dim=8, state_dim=16, ring_len=4,
                        io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=1)


def _x(w, T):
    return runs.widen_inputs(synth.step_inputs(w, 0, T), w.io_dtype)


def _S0(w):
    return np.zeros((w.batch, w.heads, w.head_dim, w.state_dim))


def test_verify_all_accepted_equals_standard():
    W, R = 3, 4
    x = _x(W_TINY, R * W)
    S_std = _S0(W_TINY)
    y_std = runs.standard(x, S_std)
    S_ver = _S0(W_TINY)
    y_ver = runs.verify_rounds(x, np.full((R, W_TINY.batch), W), W, S_ver)
    assert np.allclose(y_ver.reshape(R * W, *y_ver.shape[2:]), y_std, rtol=1e-13, atol=1e-13)
    assert np.allclose(S_ver, S_std, rtol=1e-13, atol=1e-13)


def test_verify_none_accepted_keeps_state():
    W, R = 2, 3
    x = _x(W_TINY, R * W)
    S = np.random.default_rng(1).standard_normal((3, 4, 8, 16))
    S_keep = S.copy()
    y = runs.verify_rounds(x, np.zeros((R, 3), dtype=int), W, S)
    assert np.array_equal(S, S_keep)
    # every round scores its drafts from the same untouched state
    for r in range(R):
        Sr = S_keep.copy()
        rows = {k: v[r * W:(r + 1) * W] for k, v in x.items()}
        assert np.allclose(y[r], runs.standard(rows, Sr), rtol=1e-13, atol=1e-13)


def test_verify_state_equals_accepted_prefix_replay():
    W, R = 4, 5
    x = _x(W_TINY, R * W)
    acc = synth.accept_counts(W_TINY, R, W)
    S = _S0(W_TINY)
    runs.verify_rounds(x, acc, W, S)
    for b in range(W_TINY.batch):
        keep = [r * W + i for r in range(R) for i in range(acc[r, b])]
        xb = {k: v[keep][:, [b]] for k, v in x.items()}
        Sb = _S0(W_TINY)[[b]].copy()
        runs.standard(xb, Sb)
        assert np.allclose(S[b], Sb[0], rtol=1e-12, atol=1e-14)


def test_dual_precision_limits():
    T, L = 12, 4
    x = _x(W_TINY, T)
    y_exact = runs.standard(x, _S0(W_TINY))
    # float32 "copy": differs from exact only by float32 rounding of the state
    y_f32 = runs.separated(x, _S0(W_TINY), L, "f32")
    assert np.max(runs.normwise_rel_err(y_f32, y_exact)) < 1e-6
    # no flush before T: shared == separated (both read the initial copy)
    S_init = np.random.default_rng(2).standard_normal((3, 4, 8, 16)) * 0.5
    for fmt in ("bf16", "fp8"):
        ysep = runs.separated(x, S_init.copy(), T, fmt)
        ysh = runs.shared(x, S_init.copy(), T, fmt)
        assert np.array_equal(ysep, ysh)
    # separated copies stay within their formats' rounding of exact outputs
    y_b = runs.separated(x, _S0(W_TINY), L, "bf16")
    y_8 = runs.separated(x, _S0(W_TINY), L, "fp8")
    assert np.max(runs.normwise_rel_err(y_b, y_exact)) < 2e-2
    assert np.max(runs.normwise_rel_err(y_8, y_exact)) < 6e-2
    # the rounding does change something (the copy path is really used)
    assert np.max(runs.normwise_rel_err(y_8, y_exact)) > 1e-4


def test_shared_rounding_enters_later_updates():
    # with slow decay the shared copy's rounding compounds, the separated
    # copy's does not: shared error exceeds separated error late in the run
    w = synth.Workload(batch=2, heads=4, groups=2, head_dim=8, state_dim=16, ring_len=4,
                       io_dtype="bf16", config=synth.CONFIG_ID["misc"], layer=2, dt_scale=0.01)
    T, L = 128, 4
    x = _x(w, T)
    S_init = np.random.default_rng(3).standard_normal((2, 4, 8, 16))
    y_exact = runs.standard(x, S_init.copy())
    for fmt in ("bf16", "fp8"):
        e_sep = runs.normwise_rel_err(runs.separated(x, S_init.copy(), L, fmt), y_exact)
        e_sh = runs.normwise_rel_err(runs.shared(x, S_init.copy(), L, fmt), y_exact)
        # same error before the first flush, larger shared error later on
        assert np.array_equal(e_sep[:L], e_sh[:L])
        assert e_sh[T // 2:].mean() > 1.5 * e_sep[T // 2:].mean()


def test_normwise_rel_err():
    y = np.array([[1.0, 2.0], [0.0, 0.0]])
    ref = np.array([[1.0, 4.0], [0.0, 0.0]])
    assert runs.normwise_rel_err(y, ref, axes=(-1,)).tolist() == [0.5, 0.0]
    assert runs.normwise_rel_err(y, ref) == 0.5


def test_verify_rounds_copy_limits():
    """The copy emulation under speculative rounds: with a copy that only
    rounds the state to float32 it reproduces the exact rounds (to that
    rounding), at ring lengths that fold every round or rarely; with the FP4
    copy and a zero start it equals the exact rounds until the first fold."""
    W, R = 3, 8
    x = _x(W_TINY, R * W)
    acc = synth.accept_counts(W_TINY, R, W)
    y_exact = runs.verify_rounds(x, acc, W, _S0(W_TINY))
    for L in (3, 4, 8, 32):
        y32 = runs.verify_rounds_copy(x, acc, W, _S0(W_TINY), L, "f32")
        assert float(np.max(runs.normwise_rel_err(y32, y_exact))) <= 1e-6, L
    y4 = runs.verify_rounds_copy(x, acc, W, _S0(W_TINY), 32, "fp4")      # never folds: reads Q(0) = 0
    assert np.allclose(y4, y_exact, rtol=1e-13, atol=1e-15)
    y4 = runs.verify_rounds_copy(x, acc, W, _S0(W_TINY), 4, "fp4")
    assert float(np.max(runs.normwise_rel_err(y4, y_exact))) > 1e-3   # folded states are read rounded


def test_copy_emulations_gated_delta_rule():
    """The copy emulations under the gated delta rule: a copy that only
    rounds the state to float32 reproduces the exact run (to that rounding)
    in standard decode and speculative rounds; shared and separated agree
    before the first flush; an e4m3 copy's rounding is really applied."""
    w = W_TINY
    T, L = 12, 4
    x = runs.widen_inputs(synth.gdn_inputs(w, 0, T), w.io_dtype)
    y_exact = runs.standard(x, _S0(w), rule="gdn")
    y32 = runs.separated(x, _S0(w), L, "f32", rule="gdn")
    assert float(np.max(runs.normwise_rel_err(y32, y_exact))) < 1e-6
    S_init = np.random.default_rng(4).standard_normal((3, 4, 8, 16)) * 0.5
    for fmt in ("bf16", "fp8", "fp4"):
        ysep = runs.separated(x, S_init.copy(), T, fmt, rule="gdn")
        ysh = runs.shared(x, S_init.copy(), T, fmt, rule="gdn")
        assert np.array_equal(ysep, ysh)
    y8 = runs.separated(x, _S0(w), L, "fp8", rule="gdn")
    assert 1e-4 < float(np.max(runs.normwise_rel_err(y8, y_exact))) < 6e-2
    # the rule really is the gated delta rule: the Mamba-2 emulation differs
    assert float(np.max(runs.normwise_rel_err(runs.separated(x, _S0(w), L, "f32"), y_exact))) > 1e-2
    W, R = 3, 6
    xv = runs.widen_inputs(synth.gdn_inputs(w, 0, R * W), w.io_dtype)
    acc = synth.accept_counts(w, R, W)
    yv = runs.verify_rounds(xv, acc, W, _S0(w), rule="gdn")
    for Lv in (3, 4, 8):
        y32v = runs.verify_rounds_copy(xv, acc, W, _S0(w), Lv, "f32", rule="gdn")
        assert float(np.max(runs.normwise_rel_err(y32v, yv))) <= 1e-6, Lv
