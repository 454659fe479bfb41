"""Call schedules run through the float64 eager oracle -- test infrastructure.

Every schedule is the plain eager recurrence fed the tokens the schedule
keeps; the ring and the checkpoint never appear (the pages state the
rewriting does not change the result: page "ReplaySSM: Cachear Inputs, No
Estado", sections "La solucion" and "Conclusion").

* standard decode: one token per step, output y_t = S_t q_t.  Every
  schedule takes rule="ssd" (Mamba-2) or rule="gdn" (the gated delta rule).
* speculative verify (same page, section "Como funciona en la practica",
  "Rollback" and "Paralelismo"; abstract page, Abstract): a round drafts W
  tokens, all W outputs are produced from the state before the round, and
  the state then keeps only the first c accepted drafts (c in 0..W; the
  rejected W-c are dropped).  Reading taken: no bonus token; every one of the
  W outputs is compared, rejected drafts' included.
* dual precision (abstract page, Abstract; page "The SSM Layer Nobody Made
  Fast (Until Now)", key technical takeaways): a low-precision copy of the
  checkpoint serves outputs.  ``separated``: the exact state keeps evolving
  and the copy is refreshed from it at every flush, so copy rounding never
  enters later updates.  ``shared``: the low-precision copy is the only
  checkpoint, so each flush starts from the rounded state.  Flushes happen
  after every L-th token (standard decode schedule).  The copy is produced
  from the state rounded to float32, as the checkpoint that takes the
  updates is float32.

Parity: standard / verify are pinned through ``core.eager``; the
dual-precision emulations are pinned by their limits (a copy format that
rounds nothing reproduces ``standard``; shared == separated when L >= T) in
tests/test_oracle_runs.py.
"""
from __future__ import annotations

import numpy as np

from . import core


def widen_inputs(inp: dict, io_dtype: str) -> dict:
    """Storage arrays from ``synth.step_inputs`` -> float64 arrays."""
    return {
        "q": core.widen(inp["q"], io_dtype),
        "k": core.widen(inp["k"], io_dtype),
        "v": core.widen(inp["v"], io_dtype),
        "dt": np.asarray(inp["dt"], dtype=np.float64),
        "a": np.asarray(inp["a"], dtype=np.float64),
    }


def _rows(x: dict, t0: int, t1: int, seqs=None) -> dict:
    if seqs is None:
        return {k: v[t0:t1] for k, v in x.items()}
    return {k: v[t0:t1][:, seqs] for k, v in x.items()}


def _eager(rule: str):
    """The eager recurrence of a layer type: "ssd" (Mamba-2, core.eager) or
    "gdn" (the gated delta rule, core.eager_gdn; dt slot beta, a slot alpha)."""
    return {"ssd": core.eager, "gdn": core.eager_gdn}[rule]


def standard(x: dict, S: np.ndarray, rule: str = "ssd") -> np.ndarray:
    """Eager over all rows of x; S float64 [B][H][P][N] updated in place."""
    return _eager(rule)(S, x["q"], x["k"], x["v"], x["dt"], x["a"])


def verify_rounds(x: dict, accept: np.ndarray, W: int, S: np.ndarray, rule: str = "ssd") -> np.ndarray:
    """Rounds of W drafts.  x holds R*W rows (round r uses rows rW..rW+W-1),
    accept int [R][B] accepted drafts per round and sequence.
    Returns y float64 [R][W][B][H][P]; S ends as the state after the
    accepted prefix of every round."""
    eager = _eager(rule)
    R = accept.shape[0]
    B, H, P, N = S.shape
    y = np.empty((R, W, B, H, P))
    for r in range(R):
        rows = _rows(x, r * W, r * W + W)
        S_try = S.copy()
        y[r] = eager(S_try, rows["q"], rows["k"], rows["v"], rows["dt"], rows["a"])
        for c in range(0, W + 1):
            sel = np.nonzero(accept[r] == c)[0]
            if len(sel) == 0 or c == 0:
                continue
            if c == W:
                S[sel] = S_try[sel]
                continue
            Sc = np.ascontiguousarray(S[sel])
            sub = {k: v[:c][:, sel] for k, v in rows.items()}
            eager(Sc, sub["q"], sub["k"], sub["v"], sub["dt"], sub["a"])
            S[sel] = Sc
    return y


def quant_dequant(S: np.ndarray, fmt: str) -> np.ndarray:
    """float64 state -> float32 -> storage codes -> float64 values."""
    s32 = S.astype(np.float32)
    if fmt == "f32":
        return s32.astype(np.float64)
    if fmt == "bf16":
        return core.bf16_decode(core.bf16_encode(s32)).astype(np.float64)
    if fmt == "fp8":
        codes, scale = core.quant_heads_e4m3(s32)
        return core.e4m3_decode(codes).astype(np.float64) * scale.astype(np.float64)[..., None, None]
    if fmt == "fp4":
        packed, scale = core.quant_blocks_mxfp4(s32)
        return core.dequant_blocks_mxfp4(packed, scale, s32.shape).astype(np.float64)
    raise ValueError(fmt)


def separated(x: dict, S: np.ndarray, L: int, fmt: str, rule: str = "ssd") -> np.ndarray:
    """Outputs read from the copy of the last flushed exact state."""
    eager = _eager(rule)
    T = x["q"].shape[0]
    S_read = quant_dequant(S, fmt)
    ys = []
    for t0 in range(0, T, L):
        rows = _rows(x, t0, min(T, t0 + L))
        ys.append(eager(S_read, rows["q"], rows["k"], rows["v"], rows["dt"], rows["a"]))
        eager(S, rows["q"], rows["k"], rows["v"], rows["dt"], rows["a"])
        if t0 + L <= T:
            S_read = quant_dequant(S, fmt)
    return np.concatenate(ys, axis=0)


def shared(x: dict, S: np.ndarray, L: int, fmt: str, rule: str = "ssd") -> np.ndarray:
    """The rounded copy is the only checkpoint: every flush starts from it.
    S ends as the (unrounded) state after the last token."""
    eager = _eager(rule)
    T = x["q"].shape[0]
    S[...] = quant_dequant(S, fmt)
    ys = []
    for t0 in range(0, T, L):
        rows = _rows(x, t0, min(T, t0 + L))
        ys.append(eager(S, rows["q"], rows["k"], rows["v"], rows["dt"], rows["a"]))
        if t0 + L <= T:
            S[...] = quant_dequant(S, fmt)
    return np.concatenate(ys, axis=0)


def normwise_rel_err(y: np.ndarray, ref: np.ndarray, axes=(-2, -1)) -> np.ndarray:
    """max |y - ref| / max |ref| over `axes` (denominator floored at 1e-30).

    The default reduces over the last two axes, (heads, P): one token's whole
    layer output for one sequence.  axes=(-1,) gives the per-head vector."""
    num = np.max(np.abs(np.asarray(y, dtype=np.float64) - ref), axis=axes)
    den = np.maximum(np.max(np.abs(ref), axis=axes), 1e-30)
    return num / den


def verify_rounds_copy(x: dict, accept: np.ndarray, W: int, S0: np.ndarray, L: int, fmt: str,
                       rule: str = "ssd") -> np.ndarray:
    """Speculative rounds whose outputs read a low-precision copy of the last
    flushed state (separated precisions), per sequence: before each round a
    ring holding >= L-W+1 accepted tokens is folded into the exact state;
    the round's W outputs come from the copy of that state followed by the
    accepted tokens since the fold and the W drafts; the accepted drafts join
    the ring.  Returns y float64 [R][W][B][H][P]."""
    eager = _eager(rule)
    R = accept.shape[0]
    B = S0.shape[0]
    H, P = x["v"].shape[2], x["v"].shape[3]
    y = np.empty((R, W, B, H, P))
    for b in range(B):
        S_fl = S0[b:b + 1].astype(np.float64).copy()
        live = []
        for r in range(R):
            if len(live) >= L - W + 1:
                sub = {k: v[live][:, b:b + 1] for k, v in x.items()}
                eager(S_fl, sub["q"], sub["k"], sub["v"], sub["dt"], sub["a"])
                live = []
            Sq = np.ascontiguousarray(quant_dequant(S_fl, fmt))
            rows = live + [r * W + i for i in range(W)]
            sub = {k: v[rows][:, b:b + 1] for k, v in x.items()}
            yy = eager(Sq, sub["q"], sub["k"], sub["v"], sub["dt"], sub["a"])
            y[r, :, b] = yy[len(live):, 0]
            live += [r * W + i for i in range(int(accept[r, b]))]
    return y
