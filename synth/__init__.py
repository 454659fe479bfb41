"""Seeded synthetic inputs for the ReplaySSM decode path.

This module is the one place that both the HIP path (through the tests and
bench.py) and the CPU oracle take their inputs from.  It holds random draws
and storage rounding only -- no step of the method.

Generator
---------
Counter-based SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014): element ``i`` of a stream with key ``K`` is
``mix64(K + (i + 1) * 0x9E3779B97F4A7C15)``.  Uniforms take the top 53 bits,
``(u >> 11) + 0.5`` times 2^-53, so they lie strictly inside (0, 1).  Normals
use Box-Muller on the uniform pair (2m, 2m+1): even indices take the cosine
branch and odd indices the sine branch.  Because every element is a pure
function of (key, index), any slice of a tensor (a few sequences of a large
batch, one step of a long run) is generated on its own and equals the same
slice of the whole tensor.

Keys: ``mix64(config * 2**32 + layer * 2**8 + tensor)`` with the tensor ids in
``TENSOR``.

Value distributions (the tiny single-layer workload of the task states them;
every workload here uses them):
  q, k ~ N(0, 1/N)   v ~ N(0, 1)   dt = softplus(x), x ~ N(0, 1)
  A_h = -exp(u), u ~ U(0, 1), one per (layer, head), constant over batch/time
  a = exp(dt * A_h), evaluated in float64 from the stored float32 dt and
  rounded once to float32.
q, k, v are rounded once to the storage dtype ("f32" or "bf16", round to
nearest even); dt and a are float32.  bf16 tensors are returned as their raw
16-bit patterns (numpy uint16).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR = {"A": 0, "q": 1, "k": 2, "v": 3, "dt": 4, "accept": 5, "S0": 6, "beta": 7}

# workload ids used in the keys (one per named workload)
CONFIG_ID = {"tiny": 0, "decode": 1, "verify": 2, "dual": 3, "stacked": 4, "gdn": 5, "misc": 9}


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def mix64_scalar(x: int) -> int:
    return int(_mix64(np.array([x & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0])


def stream_key(config: int, layer: int, tensor: str) -> int:
    return mix64_scalar(config * (1 << 32) + layer * (1 << 8) + TENSOR[tensor])


def _u64(key: int, idx: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx.astype(np.uint64) + np.uint64(1)) * GAMMA
    return _mix64(z)


def uniform(key: int, idx: np.ndarray) -> np.ndarray:
    """float64 uniforms in (0, 1) at the given stream indices."""
    u = _u64(key, idx) >> np.uint64(11)
    return (u.astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal_block(key: int, idx: np.ndarray) -> np.ndarray:
    idx = idx.astype(np.uint64)
    pair = idx >> np.uint64(1)
    u1 = uniform(key, pair * np.uint64(2))
    u2 = uniform(key, pair * np.uint64(2) + np.uint64(1))
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * math.pi) * u2
    odd = (idx & np.uint64(1)).astype(bool)
    return np.where(odd, r * np.sin(th), r * np.cos(th))


_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))
    return _POOL


def normal(key: int, idx: np.ndarray) -> np.ndarray:
    """float64 standard normals at the given stream indices (any shape)."""
    flat = np.ascontiguousarray(idx).reshape(-1)
    n = flat.size
    if n < (1 << 20):
        out = _normal_block(key, flat)
    else:
        chunk = 1 << 18
        parts = [flat[i:i + chunk] for i in range(0, n, chunk)]
        out = np.concatenate(list(_pool().map(lambda p: _normal_block(key, p), parts)))
    return out.reshape(np.shape(idx))


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> bf16 bit patterns (uint16), via float32 then torch's
    round-to-nearest-even conversion (storage rounding of generated inputs)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def store(x: np.ndarray, io_dtype: str) -> np.ndarray:
    if io_dtype == "f32":
        return x.astype(np.float32)
    if io_dtype == "bf16":
        return round_bf16_bits(x)
    raise ValueError(io_dtype)


@dataclass(frozen=True)
class Workload:
    """Shape of one SSM layer's decode state, plus the keys' identity."""
    batch: int
    heads: int
    groups: int
    head_dim: int      # P
    state_dim: int     # N
    ring_len: int      # L
    io_dtype: str = "bf16"
    config: int = CONFIG_ID["misc"]
    layer: int = 0
    dt_scale: float = 1.0   # multiplies dt before a = exp(dt*A); 1.0 is the plain recipe

    def key(self, tensor: str) -> int:
        return stream_key(self.config, self.layer, tensor)


def _flat_index(sizes, sel):
    """Row-major flat index over full `sizes` for the Cartesian product of the
    per-axis selections `sel` (each a 1-D int array)."""
    idx = np.zeros([len(s) for s in sel], dtype=np.uint64)
    mult = 1
    for ax in range(len(sizes) - 1, -1, -1):
        shape = [1] * len(sizes)
        shape[ax] = len(sel[ax])
        idx += (np.asarray(sel[ax], dtype=np.uint64) * np.uint64(mult)).reshape(shape)
        mult *= sizes[ax]
    return idx


def decay_A(w: Workload) -> np.ndarray:
    """A_h = -exp(u), u ~ U(0,1): float64 [H]."""
    return -np.exp(uniform(w.key("A"), np.arange(w.heads, dtype=np.uint64)))


def step_inputs(w: Workload, t0: int, t1: int, seqs=None) -> dict:
    """Inputs of tokens t0..t1-1 (absolute token-stream rows) for the chosen
    sequences (default: all).  Returns storage arrays:
      q, k : [T][b][G][N]   v : [T][b][H][P]   dt, a : [T][b][H] float32
    The full-batch row-major index is used for every element, so a subset of
    sequences equals the same rows of the whole batch."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    ts = np.arange(t0, t1, dtype=np.int64)
    bs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    Tn = 1 << 40  # time axis is unbounded; index = t*(B*...) + ...
    iq = _flat_index([Tn, B, G, N], [ts, bs, np.arange(G), np.arange(N)])
    q = normal(w.key("q"), iq) * math.sqrt(1.0 / N)
    k = normal(w.key("k"), iq) * math.sqrt(1.0 / N)
    iv = _flat_index([Tn, B, H, P], [ts, bs, np.arange(H), np.arange(P)])
    v = normal(w.key("v"), iv)
    idt = _flat_index([Tn, B, H], [ts, bs, np.arange(H)])
    x = normal(w.key("dt"), idt)
    # softplus, times the optional scale, rounded once to float32
    dt32 = (np.logaddexp(0.0, x) * w.dt_scale).astype(np.float32)
    A = decay_A(w)
    a32 = np.exp(dt32.astype(np.float64) * A[None, None, :]).astype(np.float32)
    return {
        "q": store(q, w.io_dtype),
        "k": store(k, w.io_dtype),
        "v": store(v, w.io_dtype),
        "dt": dt32,
        "a": a32,
    }


def accept_counts(w: Workload, rounds: int, W: int, r0: int = 0) -> np.ndarray:
    """Accepted drafts per (round, sequence) ~ Uniform{0..W}: int32 [R][B]."""
    idx = _flat_index([1 << 40, w.batch], [np.arange(r0, r0 + rounds), np.arange(w.batch)])
    u = uniform(w.key("accept"), idx)
    return np.minimum((u * (W + 1)).astype(np.int64), W).astype(np.int32)


def checkpoint_state(w: Workload, scale: float = 1.0, seqs=None) -> np.ndarray:
    """A float32 checkpoint [b][H][P][N] ~ scale * N(0, 1), e.g. a state that
    a prefill handed over."""
    B, H, P, N = w.batch, w.heads, w.head_dim, w.state_dim
    bs = np.arange(B) if seqs is None else np.asarray(seqs)
    idx = _flat_index([B, H, P, N], [bs, np.arange(H), np.arange(P), np.arange(N)])
    return (normal(w.key("S0"), idx) * scale).astype(np.float32)


def named(name: str, **over) -> Workload:
    """The workloads the task names, by what they are."""
    base = {
        # tiny single layer: B=1 H=4 G=1 P=16 N=16 L=4, all float32
        "tiny": dict(batch=1, heads=4, groups=1, head_dim=16, state_dim=16, ring_len=4, io_dtype="f32"),
        # Mamba-2-shaped layer, standard decode: B=256 H=128 G=8 P=64 N=128 L=16, bf16 q/k/v
        "decode": dict(batch=256, heads=128, groups=8, head_dim=64, state_dim=128, ring_len=16, io_dtype="bf16"),
        # speculative verify: B=256 H=64 G=8 P=64 N=128 L=16, W=5
        "verify": dict(batch=256, heads=64, groups=8, head_dim=64, state_dim=128, ring_len=16, io_dtype="bf16"),
        # dual precision: decode shapes, 1024 steps
        "dual": dict(batch=256, heads=128, groups=8, head_dim=64, state_dim=128, ring_len=16, io_dtype="bf16"),
        # stacked sweep: 8 layers, B=512 H=64 G=8 P=128 N=128, L in {8,16,32}
        "stacked": dict(batch=512, heads=64, groups=8, head_dim=128, state_dim=128, ring_len=16, io_dtype="bf16"),
        # Gated DeltaNet layer (the pages give no shape): 32 value heads over 16 key heads,
        # P = N = 128, B=256, L=16, bf16 q/k/v (gdn_inputs)
        "gdn": dict(batch=256, heads=32, groups=16, head_dim=128, state_dim=128, ring_len=16, io_dtype="bf16"),
    }[name]
    base.update(over)
    base.setdefault("config", CONFIG_ID[name])
    return Workload(**base)


def dyadic_inputs(w: Workload, t0: int, t1: int, seqs=None) -> dict:
    """Inputs whose every product and sum in the recurrence is exact in
    float32 for short runs: a in {1, 1/2}, dt in {1, 2}, v integers in
    [-4, 4], k and q one-hot.  Same layout and storage as step_inputs."""
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    ts = np.arange(t0, t1, dtype=np.int64)
    bs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    Tn = 1 << 40
    ig = _flat_index([Tn, B, G], [ts, bs, np.arange(G)])
    hot_q = np.minimum((uniform(w.key("q"), ig) * N).astype(np.int64), N - 1)
    hot_k = np.minimum((uniform(w.key("k"), ig) * N).astype(np.int64), N - 1)
    q = (np.arange(N) == hot_q[..., None]).astype(np.float64)
    k = (np.arange(N) == hot_k[..., None]).astype(np.float64)
    iv = _flat_index([Tn, B, H, P], [ts, bs, np.arange(H), np.arange(P)])
    v = np.floor(uniform(w.key("v"), iv) * 9.0) - 4.0
    ih = _flat_index([Tn, B, H], [ts, bs, np.arange(H)])
    u = uniform(w.key("dt"), ih)
    dt = np.where(u < 0.5, 1.0, 2.0).astype(np.float32)
    a = np.where(uniform(w.key("A"), ih) < 0.5, 1.0, 0.5).astype(np.float32)
    return {"q": store(q, w.io_dtype), "k": store(k, w.io_dtype), "v": store(v, w.io_dtype),
            "dt": dt, "a": a}


# ---------------------------------------------------------------------------
# The same recipe evaluated with torch on a device, for long full-batch runs.
# Integer steps are bit-identical to the numpy path (uint64 arithmetic done
# in int64 two's complement); the float64 transcendental functions of the
# device may differ from the host's in the last bit, so a test that feeds
# the oracle from this path copies the very device tensors back to the host.

def _s64(x: int) -> int:
    x &= 0xFFFFFFFFFFFFFFFF
    return x - (1 << 64) if x >= (1 << 63) else x


_GAMMA_S = _s64(0x9E3779B97F4A7C15)
_M1_S = _s64(0xBF58476D1CE4E5B9)
_M2_S = _s64(0x94D049BB133111EB)


def _t_srl(z, s: int):
    """logical right shift of int64 tensors"""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _t_mix64(z):
    z = z ^ _t_srl(z, 30)
    z = z * _M1_S
    z = z ^ _t_srl(z, 27)
    z = z * _M2_S
    return z ^ _t_srl(z, 31)


def _t_uniform(key: int, idx):
    z = _t_mix64(idx.mul(_GAMMA_S).add(_s64(key + _GAMMA_S)))   # key + (idx + 1) * gamma
    import torch
    return (_t_srl(z, 11).to(torch.float64) + 0.5) * (2.0 ** -53)


def _t_normal(key: int, idx):
    import torch
    pair = idx >> 1
    u1 = _t_uniform(key, pair * 2)
    u2 = _t_uniform(key, pair * 2 + 1)
    r = torch.sqrt(-2.0 * torch.log(u1))
    th = (2.0 * math.pi) * u2
    return torch.where((idx & 1).bool(), r * torch.sin(th), r * torch.cos(th))


def _t_index(sizes, sel, device):
    import torch
    idx = torch.zeros([len(s) for s in sel], dtype=torch.int64, device=device)
    mult = 1
    for ax in range(len(sizes) - 1, -1, -1):
        shape = [1] * len(sizes)
        shape[ax] = len(sel[ax])
        idx += (torch.as_tensor(np.asarray(sel[ax]), dtype=torch.int64, device=device) * mult).reshape(shape)
        mult *= sizes[ax]
    return idx


def step_inputs_torch(w: Workload, t0: int, t1: int, device="cuda") -> dict:
    """step_inputs evaluated on `device`; q, k, v come back as torch
    bfloat16 / float32 tensors, dt and a as float32."""
    import torch
    B, H, G, P, N = w.batch, w.heads, w.groups, w.head_dim, w.state_dim
    ts, bs = np.arange(t0, t1), np.arange(B)
    Tn = 1 << 40
    iq = _t_index([Tn, B, G, N], [ts, bs, np.arange(G), np.arange(N)], device)
    q = _t_normal(w.key("q"), iq) * math.sqrt(1.0 / N)
    k = _t_normal(w.key("k"), iq) * math.sqrt(1.0 / N)
    del iq
    iv = _t_index([Tn, B, H, P], [ts, bs, np.arange(H), np.arange(P)], device)
    v = _t_normal(w.key("v"), iv)
    del iv
    idt = _t_index([Tn, B, H], [ts, bs, np.arange(H)], device)
    x = _t_normal(w.key("dt"), idt)
    dt32 = (torch.nn.functional.softplus(x) * w.dt_scale).to(torch.float32)
    A = torch.as_tensor(decay_A(w), dtype=torch.float64, device=device)
    a32 = torch.exp(dt32.to(torch.float64) * A).to(torch.float32)
    io = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    return {"q": q.to(torch.float32).to(io), "k": k.to(torch.float32).to(io),
            "v": v.to(torch.float32).to(io), "dt": dt32, "a": a32}


def gdn_inputs(w: Workload, t0: int, t1: int, seqs=None) -> dict:
    """Inputs of a Gated DeltaNet layer, same layout and streams as
    step_inputs: q and k are the step_inputs draws scaled to unit length per
    (token, sequence, group) row (in float64, then stored); v as
    step_inputs; the dt slot carries beta = sigmoid(x), x ~ N(0, 1) (stream
    "beta"), and the a slot the step_inputs decay a in (0, 1) as alpha."""
    x = step_inputs(w, t0, t1, seqs)
    out = dict(x)
    for name in ("q", "k"):
        raw = _unstore(x[name], w.io_dtype)
        out[name] = store(raw / np.linalg.norm(raw, axis=-1, keepdims=True), w.io_dtype)
    B, H = w.batch, w.heads
    ts = np.arange(t0, t1, dtype=np.int64)
    bs = np.arange(B, dtype=np.int64) if seqs is None else np.asarray(seqs, dtype=np.int64)
    ib = _flat_index([1 << 40, B, H], [ts, bs, np.arange(H)])
    out["dt"] = (1.0 / (1.0 + np.exp(-normal(w.key("beta"), ib)))).astype(np.float32)
    return out


def _unstore(x: np.ndarray, io_dtype: str) -> np.ndarray:
    """Storage array -> float64 values (bf16 patterns widened)."""
    if io_dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def gdn_inputs_torch(w: Workload, t0: int, t1: int, device="cuda") -> dict:
    """gdn_inputs evaluated on `device` (as step_inputs_torch)."""
    import torch
    x = step_inputs_torch(w, t0, t1, device)
    out = dict(x)
    for name in ("q", "k"):
        raw = x[name].to(torch.float64)
        out[name] = (raw / torch.linalg.vector_norm(raw, dim=-1, keepdim=True)).to(torch.float32).to(x[name].dtype)
    B, H = w.batch, w.heads
    ib = _t_index([1 << 40, B, H], [np.arange(t0, t1), np.arange(B), np.arange(H)], device)
    out["dt"] = torch.sigmoid(_t_normal(w.key("beta"), ib)).to(torch.float32)
    return out


def to_storage(t) -> np.ndarray:
    """A device tensor from step_inputs_torch -> the numpy storage array the
    oracle widens (bf16 as uint16 patterns)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
