"""ctypes front of the float64 C oracle (``replay_oracle.c``) -- test
infrastructure only.

Pinned by tests/test_oracle_pins.py (eager recurrence: history form, causal
linear attention, decay special cases, the masked-matrix form, linearity,
group sharing, a hand-worked example) and tests/test_oracle_quant.py
(quantisers: torch's CPU float conversions, the E4M3 format's own table,
saturation and tie cases).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "replay_oracle.c")
_SO = os.path.join(_HERE, "_replay_oracle.so")
_LOCK = threading.Lock()
_LIB = None

_F64P = ctypes.POINTER(ctypes.c_double)
_F32P = ctypes.POINTER(ctypes.c_float)
_U16P = ctypes.POINTER(ctypes.c_uint16)
_U8P = ctypes.POINTER(ctypes.c_uint8)
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile replay_oracle.c into _replay_oracle.so (gcc, OpenMP, IEEE)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            build(force=False)
            L = ctypes.CDLL(_SO)
            L.oracle_eager.argtypes = [_I64] * 6 + [_F64P] * 7
            L.oracle_eager.restype = None
            L.oracle_eager_gdn.argtypes = [_I64] * 6 + [_F64P] * 7
            L.oracle_eager_gdn.restype = None
            L.oracle_threads.restype = ctypes.c_int
            L.oracle_set_threads.argtypes = [ctypes.c_int]
            L.oracle_bf16_encode_n.argtypes = [_F32P, _U16P, _I64]
            L.oracle_bf16_decode_n.argtypes = [_U16P, _F32P, _I64]
            L.oracle_e4m3_encode_n.argtypes = [_F32P, _U8P, _I64]
            L.oracle_e4m3_decode_n.argtypes = [_U8P, _F32P, _I64]
            L.oracle_quant_heads_e4m3.argtypes = [_F32P, _I64, _I64, _U8P, _F32P]
            L.oracle_e2m1_decode_n.argtypes = [_U8P, _F32P, _I64]
            L.oracle_e2m1_encode_n.argtypes = [_F64P, _U8P, _I64]
            L.oracle_quant_blocks_mxfp4.argtypes = [_F32P, _I64, _U8P, _U8P]
            L.oracle_dequant_blocks_mxfp4.argtypes = [_U8P, _U8P, _I64, _F32P]
            _LIB = L
    return _LIB


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for later oracle calls (a timing knob; the results do not depend on it)."""
    lib().oracle_set_threads(int(n))


def _p(a, t):
    return a.ctypes.data_as(t)


def bf16_decode(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint16)
    out = np.empty(c.shape, dtype=np.float32)
    lib().oracle_bf16_decode_n(_p(c, _U16P), _p(out, _F32P), c.size)
    return out


def bf16_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_encode_n(_p(x, _F32P), _p(out, _U16P), x.size)
    return out


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().oracle_e4m3_decode_n(_p(c, _U8P), _p(out, _F32P), c.size)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_n(_p(x, _F32P), _p(out, _U8P), x.size)
    return out


def quant_heads_e4m3(x: np.ndarray):
    """x: float32 [..., P, N] -> (codes uint8 same shape, scale float32 [...])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:-2]
    heads = int(np.prod(lead)) if lead else 1
    n = x.shape[-1] * x.shape[-2]
    codes = np.empty(x.shape, dtype=np.uint8)
    scale = np.empty(lead, dtype=np.float32)
    lib().oracle_quant_heads_e4m3(_p(x, _F32P), heads, n, _p(codes, _U8P), _p(scale, _F32P))
    return codes, scale


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    """4-bit codes (low nibble of each byte) -> float32 values."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().oracle_e2m1_decode_n(_p(c, _U8P), _p(out, _F32P), c.size)
    return out


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """float64 values -> 4-bit codes (nearest, ties to even, saturating)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e2m1_encode_n(_p(x, _F64P), _p(out, _U8P), x.size)
    return out


def quant_blocks_mxfp4(x: np.ndarray):
    """x: float32 [..., P, N] (P*N a multiple of 32) -> (packed codes uint8
    [..., P*N/2], E8M0 scales uint8 [..., P*N/32]); blocks of 32 consecutive
    values of each head's row-major tile."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:-2]
    n = x.shape[-1] * x.shape[-2]
    assert n % 32 == 0
    nblk = x.size // 32
    packed = np.empty(lead + (n // 2,), dtype=np.uint8)
    scale = np.empty(lead + (n // 32,), dtype=np.uint8)
    lib().oracle_quant_blocks_mxfp4(_p(x, _F32P), nblk, _p(packed, _U8P), _p(scale, _U8P))
    return packed, scale


def dequant_blocks_mxfp4(packed: np.ndarray, scale: np.ndarray, shape) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint8)
    out = np.empty(shape, dtype=np.float32)
    lib().oracle_dequant_blocks_mxfp4(_p(packed, _U8P), _p(scale, _U8P), scale.size, _p(out, _F32P))
    return out


def widen(arr: np.ndarray, io_dtype: str) -> np.ndarray:
    """Stored input values -> exact float64 (bf16 patterns are decoded)."""
    if io_dtype == "bf16":
        return bf16_decode(arr).astype(np.float64)
    return np.asarray(arr).astype(np.float64)


def eager(S: np.ndarray, q, k, v, dt, a) -> np.ndarray:
    """Run the eager recurrence in float64 over T tokens.

    S  : float64 [B][H][P][N], updated in place (state before -> after)
    q,k: float64 [T][B][G][N]   v: [T][B][H][P]   dt, a: [T][B][H]
    returns y: float64 [T][B][H][P]
    """
    assert S.dtype == np.float64 and S.flags.c_contiguous
    T, B, G, N = q.shape
    H, P = v.shape[2], v.shape[3]
    assert S.shape == (B, H, P, N), (S.shape, (B, H, P, N))
    assert k.shape == q.shape and v.shape == (T, B, H, P)
    assert dt.shape == (T, B, H) and a.shape == (T, B, H)
    assert H % G == 0
    args = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dt, a)]
    y = np.empty((T, B, H, P), dtype=np.float64)
    if T == 0 or B == 0:
        return y
    lib().oracle_eager(T, B, H, G, P, N, *[_p(x, _F64P) for x in args], _p(S, _F64P), _p(y, _F64P))
    return y


def eager_gdn(S: np.ndarray, q, k, v, beta, alpha) -> np.ndarray:
    """Run the gated delta rule (replay_oracle.c oracle_eager_gdn) in float64
    over T tokens: S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    y_t = S_t q_t.  Shapes as eager(), beta and alpha in the dt and a slots.
    The pages name Gated DeltaNet without its equation; this is the published
    rule (Yang et al., ICLR 2025), pinned by tests/test_oracle_gdn.py."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    T, B, G, N = q.shape
    H, P = v.shape[2], v.shape[3]
    assert S.shape == (B, H, P, N), (S.shape, (B, H, P, N))
    assert k.shape == q.shape and v.shape == (T, B, H, P)
    assert beta.shape == (T, B, H) and alpha.shape == (T, B, H)
    assert H % G == 0
    args = [np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, beta, alpha)]
    y = np.empty((T, B, H, P), dtype=np.float64)
    if T == 0 or B == 0:
        return y
    lib().oracle_eager_gdn(T, B, H, G, P, N, *[_p(x, _F64P) for x in args], _p(S, _F64P), _p(y, _F64P))
    return y
