"""Python binding of libreplayssm: the ReplaySSM decode path for Mamba-2-style
SSM layers on MI355X (gfx950).

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; torch supplies device memory and the current stream.  The entry
points keep the C names (``replay_init``, ``replay_append``, ...).
``ReplayLayer`` bundles one layer's buffers and handle for convenience.

If the built library is missing, importing this package raises ImportError:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "ReplayError", "ReplayConfig", "ReplayBuffers", "ReplayLayer", "lib", "LIB_PATH",
    "F32", "BF16", "FP8_E4M3", "FP4_E2M1", "NONE", "SEQERR_RING_OVERFLOW", "SEQERR_ROLLBACK_RANGE",
    "SEQERR_TOO_FEW", "SEQERR_POS_OVERFLOW", "EXPORTS",
    "replay_status_string", "replay_abi_version", "replay_buffer_bytes", "replay_init",
    "replay_destroy", "replay_load_checkpoint", "replay_append", "replay_decode",
    "replay_verify", "replay_rollback", "replay_flush", "replay_step", "replay_step_layers", "replay_step_static",
    "replay_verify_step", "replay_rollback_verify_step", "replay_set_flush_skipping", "replay_get_error",
    "replay_eager_step", "replay_eager_select", "replay_stream_probe",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libreplayssm.so")

NONE, F32, BF16, FP8_E4M3, FP4_E2M1 = -1, 0, 1, 2, 3
SEQERR_RING_OVERFLOW, SEQERR_ROLLBACK_RANGE, SEQERR_TOO_FEW, SEQERR_POS_OVERFLOW = 1, 2, 4, 8

# every symbol include/replayssm.h declares
EXPORTS = (
    "replay_status_string", "replay_abi_version", "replay_buffer_bytes", "replay_init",
    "replay_destroy", "replay_load_checkpoint", "replay_append", "replay_decode",
    "replay_verify", "replay_rollback", "replay_flush", "replay_step", "replay_step_layers", "replay_step_static",
    "replay_verify_step", "replay_rollback_verify_step", "replay_set_flush_skipping", "replay_get_error",
    "replay_eager_step", "replay_eager_select", "replay_stream_probe",
)

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32


class ReplayConfig(ctypes.Structure):
    _fields_ = [("batch", _I32), ("heads", _I32), ("groups", _I32), ("head_dim", _I32),
                ("state_dim", _I32), ("ring_len", _I32), ("io_dtype", _I32),
                ("read_copy", _I32), ("shared_lowp", _I32), ("rule", _I32)]


BUFFER_FIELDS = ("s_master", "s_copy", "s_scale", "ring_q", "ring_k", "ring_v", "ring_dt",
                 "ring_a", "pos", "base", "err", "sync")


class ReplayBuffers(ctypes.Structure):
    _fields_ = [(name, _VP) for name in BUFFER_FIELDS]


class ReplayError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.replay_status_string.argtypes = [ctypes.c_int]
    L.replay_status_string.restype = ctypes.c_char_p
    L.replay_abi_version.restype = _I32
    L.replay_buffer_bytes.argtypes = [ctypes.POINTER(ReplayConfig), ctypes.POINTER(ctypes.c_size_t)]
    L.replay_init.argtypes = [ctypes.POINTER(ReplayConfig), ctypes.POINTER(ReplayBuffers), _VP,
                              ctypes.POINTER(_VP)]
    L.replay_destroy.argtypes = [_VP, _VP]
    L.replay_load_checkpoint.argtypes = [_VP, _VP, _VP]
    L.replay_append.argtypes = [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]
    L.replay_decode.argtypes = [_VP, _VP, _VP]
    L.replay_verify.argtypes = [_VP, _I32, _VP, _VP]
    L.replay_rollback.argtypes = [_VP, _VP, _VP]
    L.replay_flush.argtypes = [_VP, _I32, _VP]
    L.replay_step.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]
    L.replay_verify_step.argtypes = [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]
    L.replay_rollback_verify_step.argtypes = [_VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]
    L.replay_get_error.argtypes = [_VP, ctypes.POINTER(_I32), _VP, _VP]
    L.replay_set_flush_skipping.argtypes = [_VP, _I32, _VP]
    L.replay_step_static.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]
    L.replay_step_layers.argtypes = [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]
    L.replay_eager_step.argtypes = [ctypes.POINTER(ReplayConfig)] + [_VP] * 9
    L.replay_eager_select.argtypes = [ctypes.POINTER(ReplayConfig), _VP, _I32, _VP, _VP, _VP]
    L.replay_stream_probe.argtypes = [_I32, _VP, _VP, ctypes.c_size_t, _VP]
    for name in EXPORTS:
        if name not in ("replay_status_string", "replay_abi_version"):
            getattr(L, name).restype = ctypes.c_int
    return L


lib = _load()


def _check(status: int, what: str):
    if status != 0:
        raise ReplayError(f"{what}: {lib.replay_status_string(status).decode()} (status {status})")


def _ptr(t):
    """Device pointer of a torch tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- the C entry points, same names --------------------------------------

def replay_status_string(status: int) -> str:
    return lib.replay_status_string(status).decode()


def replay_abi_version() -> int:
    return int(lib.replay_abi_version())


def replay_buffer_bytes(cfg: ReplayConfig):
    out = (ctypes.c_size_t * len(BUFFER_FIELDS))()
    _check(lib.replay_buffer_bytes(ctypes.byref(cfg), out), "replay_buffer_bytes")
    return dict(zip(BUFFER_FIELDS, [int(x) for x in out]))


def replay_init(cfg: ReplayConfig, bufs: ReplayBuffers, stream=None):
    h = _VP()
    _check(lib.replay_init(ctypes.byref(cfg), ctypes.byref(bufs), _stream(stream), ctypes.byref(h)),
           "replay_init")
    return h


def replay_destroy(h, stream=None):
    _check(lib.replay_destroy(h, _stream(stream)), "replay_destroy")


def replay_load_checkpoint(h, s_src, stream=None):
    _check(lib.replay_load_checkpoint(h, _ptr(s_src), _stream(stream)), "replay_load_checkpoint")


def replay_append(h, W, q, k, v, dt, a, stream=None):
    _check(lib.replay_append(h, W, _ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a), _stream(stream)),
           "replay_append")


def replay_decode(h, y, stream=None):
    _check(lib.replay_decode(h, _ptr(y), _stream(stream)), "replay_decode")


def replay_verify(h, W, y, stream=None):
    _check(lib.replay_verify(h, W, _ptr(y), _stream(stream)), "replay_verify")


def replay_rollback(h, n_reject, stream=None):
    _check(lib.replay_rollback(h, _ptr(n_reject), _stream(stream)), "replay_rollback")


def replay_flush(h, min_count, stream=None):
    _check(lib.replay_flush(h, min_count, _stream(stream)), "replay_flush")


def replay_step(h, q, k, v, dt, a, y, flush_at, stream=None):
    _check(lib.replay_step(h, _ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a), _ptr(y), flush_at,
                           _stream(stream)), "replay_step")


def replay_step_layers(handles, q, k, v, dt, a, y, flush_at, stream=None):
    """handles, q, k, v, dt, a, y: sequences of n entries (one per layer)."""
    n = len(handles)
    arr = lambda xs: (_VP * n)(*[_ptr(x) for x in xs])
    _check(lib.replay_step_layers((_VP * n)(*handles), n, arr(q), arr(k), arr(v), arr(dt), arr(a), arr(y),
                                  int(flush_at), _stream(stream)), "replay_step_layers")


def replay_step_static(h, q, k, v, dt, a, y, flush_at, stream=None):
    _check(lib.replay_step_static(h, _ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a), _ptr(y), int(flush_at),
                                  _stream(stream)), "replay_step_static")


def replay_rollback_verify_step(h, n_reject, W, q, k, v, dt, a, y, flush_at, stream=None):
    _check(lib.replay_rollback_verify_step(h, _ptr(n_reject), W, _ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a),
                                           _ptr(y), flush_at, _stream(stream)), "replay_rollback_verify_step")


def replay_verify_step(h, W, q, k, v, dt, a, y, flush_at, stream=None):
    _check(lib.replay_verify_step(h, W, _ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a), _ptr(y), flush_at,
                                  _stream(stream)), "replay_verify_step")


def replay_set_flush_skipping(h, enable: int, stream=None):
    _check(lib.replay_set_flush_skipping(h, int(enable), _stream(stream)), "replay_set_flush_skipping")


def replay_get_error(h, batch: int, stream=None):
    """Returns (word, per_sequence list)."""
    word = _I32()
    per = (_I32 * batch)()
    _check(lib.replay_get_error(h, ctypes.byref(word), per, _stream(stream)), "replay_get_error")
    return int(word.value), list(per)


def replay_eager_step(cfg, s_in, s_out, q, k, v, dt, a, y, stream=None):
    _check(lib.replay_eager_step(ctypes.byref(cfg), _ptr(s_in), _ptr(s_out), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(dt), _ptr(a), _ptr(y), _stream(stream)), "replay_eager_step")


def replay_eager_select(cfg, snaps, W, n_accept, s, stream=None):
    _check(lib.replay_eager_select(ctypes.byref(cfg), _ptr(snaps), W, _ptr(n_accept), _ptr(s),
                                   _stream(stream)), "replay_eager_select")


def replay_stream_probe(mode, src, dst, nbytes, stream=None):
    _check(lib.replay_stream_probe(mode, _ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "replay_stream_probe")


# ---- one layer's state, allocated with torch -------------------------------

_DTYPE_CODE = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp4": FP4_E2M1, None: NONE, "none": NONE}
# replay_rule: the layer's recurrence ("mamba2": S = a S + dt v k^T; "gdn": the
# gated delta rule, dt carrying beta and a carrying alpha)
RULE_CODE = {"mamba2": 0, "gdn": 1}
MAMBA2, GATED_DELTA = 0, 1


class ReplayLayer:
    """Buffers + handle of one SSM layer's decode state on the current GPU.

    Tensors (torch, on `device`): s_master [B,H,P,N] f32 (absent in shared
    mode), s_copy [B,H,P,N] bf16/uint8 or [B,H,P*N/2] uint8 FP4 codes (when
    read_copy is set), s_scale [B,H] f32 (e4m3) or [B,H,P*N/32] uint8 E8M0
    (FP4), ring_q/ring_k [B,G,L,N], ring_v [B,H,L,P] (io
    dtype), ring_dt/ring_a [B,L,H] f32 (slot-major), pos/base [B] int32, err [B+1] int32,
    sync [B, G+1, 32] int32 (arrival counters, one per 128-byte line; not
    allocated with counters=False, for a layer stepped by step_static only).
    """

    def __init__(self, batch, heads, groups, head_dim, state_dim, ring_len, io_dtype="bf16",
                 read_copy=None, shared_lowp=False, device="cuda", stream=None, counters=True, rule="mamba2"):
        import torch
        self.cfg = ReplayConfig(batch, heads, groups, head_dim, state_dim, ring_len,
                                _DTYPE_CODE[io_dtype], _DTYPE_CODE[read_copy], int(bool(shared_lowp)),
                                RULE_CODE[rule])
        self.rule = rule
        self.io_dtype = io_dtype
        self.read_copy = read_copy
        nbytes = replay_buffer_bytes(self.cfg)
        B, H, G, P, N, L = batch, heads, groups, head_dim, state_dim, ring_len
        iot = torch.bfloat16 if io_dtype == "bf16" else torch.float32
        copy_t = torch.bfloat16 if read_copy == "bf16" else torch.uint8
        fp4 = read_copy == "fp4"
        shapes = {
            "s_master": ((B, H, P, N), torch.float32),
            "s_copy": ((B, H, P * N // 2) if fp4 else (B, H, P, N), copy_t),
            "s_scale": ((B, H, P * N // 32), torch.uint8) if fp4 else ((B, H), torch.float32),
            "ring_q": ((B, G, L, N), iot),
            "ring_k": ((B, G, L, N), iot), "ring_v": ((B, H, L, P), iot),
            "ring_dt": ((B, L, H), torch.float32), "ring_a": ((B, L, H), torch.float32),
            "pos": ((B,), torch.int32), "base": ((B,), torch.int32), "err": ((B + 1,), torch.int32),
            "sync": ((B, G + 1, 32), torch.int32),
        }
        self.t = {}
        for name in BUFFER_FIELDS:
            if nbytes[name] == 0 or (name == "sync" and not counters):
                self.t[name] = None
                continue
            shape, dt = shapes[name]
            t = torch.empty(shape, dtype=dt, device=device)
            assert t.numel() * t.element_size() == nbytes[name], name
            self.t[name] = t
        self.bufs = ReplayBuffers(*[_ptr(self.t[n]) for n in BUFFER_FIELDS])
        self.h = replay_init(self.cfg, self.bufs, stream)

    def __getattr__(self, name):
        t = self.__dict__.get("t")
        if t is not None and name in t:
            return t[name]
        raise AttributeError(name)

    def append(self, W, q, k, v, dt, a, stream=None):
        replay_append(self.h, W, q, k, v, dt, a, stream)

    def decode(self, y, stream=None):
        replay_decode(self.h, y, stream)

    def verify(self, W, y, stream=None):
        replay_verify(self.h, W, y, stream)

    def rollback(self, n_reject, stream=None):
        replay_rollback(self.h, n_reject, stream)

    def flush(self, min_count, stream=None):
        replay_flush(self.h, min_count, stream)

    def step(self, q, k, v, dt, a, y, flush_at=None, stream=None):
        replay_step(self.h, q, k, v, dt, a, y, self.cfg.ring_len if flush_at is None else flush_at, stream)

    def step_static(self, q, k, v, dt, a, y, flush_at=None, stream=None):
        """replay_step with the library's static arrival counters (no `sync` buffer needed)."""
        replay_step_static(self.h, q, k, v, dt, a, y, self.cfg.ring_len if flush_at is None else flush_at, stream)

    def verify_step(self, W, q, k, v, dt, a, y, flush_at=None, stream=None):
        """Fold if due (count >= flush_at, default L - W + 1), append W drafts, score them."""
        fa = self.cfg.ring_len - W + 1 if flush_at is None else flush_at
        replay_verify_step(self.h, W, q, k, v, dt, a, y, fa, stream)

    def rollback_verify_step(self, n_reject, W, q, k, v, dt, a, y, flush_at=None, stream=None):
        """rollback(n_reject), then verify_step(W, ...), fused where the round is one launch."""
        fa = self.cfg.ring_len - W + 1 if flush_at is None else flush_at
        replay_rollback_verify_step(self.h, n_reject, W, q, k, v, dt, a, y, fa, stream)

    def load_checkpoint(self, s_src, stream=None):
        replay_load_checkpoint(self.h, s_src, stream)

    def set_flush_skipping(self, enable: bool, stream=None):
        replay_set_flush_skipping(self.h, 1 if enable else 0, stream)

    def get_error(self, stream=None):
        return replay_get_error(self.h, self.cfg.batch, stream)

    def close(self, stream=None):
        if self.h is not None:
            replay_destroy(self.h, stream)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
