"""The C ABI without a GPU: the built library loads, exports every symbol
include/replayssm.h declares, and its host-only calls (status strings,
version, buffer sizing, argument validation) behave as documented.  No call
here reaches the device: every config below is rejected before any launch,
or the call is host-only."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "replayssm.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(replay_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lad():
    import linear_attention_decode_amd as m
    return m


def test_every_declared_symbol_is_exported(lad):
    names = _declared()
    assert len(names) >= 15
    raw = ctypes.CDLL(lad.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    assert set(names) == set(lad.EXPORTS)


def test_version_and_status_strings(lad):
    assert lad.replay_abi_version() == 8
    for s, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported"), (3, "HIP"), (4, "static counters")]:
        assert text in lad.replay_status_string(s)
    assert lad.replay_status_string(99) == "unknown status"


def test_buffer_bytes_match_the_layout(lad):
    c = lad.ReplayConfig(256, 128, 8, 64, 128, 16, lad.BF16, lad.NONE, 0)
    b = lad.replay_buffer_bytes(c)
    assert b["s_master"] == 256 * 128 * 64 * 128 * 4
    assert b["s_copy"] == 0 and b["s_scale"] == 0
    assert b["ring_q"] == b["ring_k"] == 256 * 8 * 16 * 128 * 2
    assert b["ring_v"] == 256 * 128 * 16 * 64 * 2
    assert b["ring_dt"] == b["ring_a"] == 256 * 128 * 16 * 4
    assert b["pos"] == b["base"] == 256 * 4 and b["err"] == 257 * 4 and b["sync"] == 256 * 9 * 128
    c8 = lad.ReplayConfig(4, 8, 2, 128, 128, 32, lad.F32, lad.FP8_E4M3, 1)
    b8 = lad.replay_buffer_bytes(c8)
    assert b8["s_master"] == 0 and b8["s_copy"] == 4 * 8 * 128 * 128 and b8["s_scale"] == 4 * 8 * 4
    assert b8["ring_v"] == 4 * 8 * 32 * 128 * 4
    c4 = lad.ReplayConfig(4, 8, 2, 64, 128, 16, lad.BF16, lad.FP4_E2M1, 0)
    b4 = lad.replay_buffer_bytes(c4)
    assert b4["s_master"] == 4 * 8 * 64 * 128 * 4
    assert b4["s_copy"] == 4 * 8 * 64 * 128 // 2 and b4["s_scale"] == 4 * 8 * 64 * 128 // 32
    c4s = lad.ReplayConfig(4, 8, 2, 64, 128, 16, lad.BF16, lad.FP4_E2M1, 1)   # shared FP4: no master
    b4s = lad.replay_buffer_bytes(c4s)
    assert b4s["s_master"] == 0
    assert b4s["s_copy"] == b4["s_copy"] and b4s["s_scale"] == b4["s_scale"]
    # a gated-delta layer with a copy holds the same buffers as a Mamba-2 layer
    for cp, sh in ((lad.FP4_E2M1, 0), (lad.FP8_E4M3, 1), (lad.BF16, 0)):
        m2 = lad.replay_buffer_bytes(lad.ReplayConfig(4, 8, 2, 64, 128, 16, lad.BF16, cp, sh))
        gd = lad.replay_buffer_bytes(lad.ReplayConfig(4, 8, 2, 64, 128, 16, lad.BF16, cp, sh, lad.GATED_DELTA))
        assert gd == m2


@pytest.mark.parametrize("fields,status", [
    ((0, 4, 1, 64, 128, 16, 1, -1, 0), 1),          # batch 0
    ((2, 6, 4, 64, 128, 16, 1, -1, 0), 1),          # H % G != 0
    ((2, 4, 1, 32, 128, 16, 1, -1, 0), 2),          # P=32 not compiled
    ((2, 4, 1, 64, 256, 16, 1, -1, 0), 2),          # N=256 not compiled
    ((2, 4, 1, 64, 128, 33, 1, -1, 0), 2),          # L > 32
    ((2, 4, 1, 64, 128, 0, 1, -1, 0), 1),           # L = 0
    ((2, 4, 1, 64, 128, 16, 2, -1, 0), 2),          # io dtype e4m3
    ((2, 4, 1, 64, 128, 16, 1, 7, 0), 2),           # unknown copy dtype
    ((2, 4, 1, 64, 128, 16, 1, -1, 1), 1),          # shared without a copy
    ((2, 4, 1, 64, 128, 16, 1, 3, 2), 1),           # shared flag neither 0 nor 1
    ((2, 4, 1, 64, 128, 16, 1, -1, 0, 2), 1),       # unknown rule
    ((2, 4, 1, 64, 128, 16, 1, -1, 1, 1), 1),       # gated delta rule, shared without a copy
])
def test_invalid_configs_are_rejected_on_the_host(lad, fields, status):
    c = lad.ReplayConfig(*fields)
    with pytest.raises(lad.ReplayError) as e:
        lad.replay_buffer_bytes(c)
    assert f"status {status}" in str(e.value)
    with pytest.raises(lad.ReplayError):
        lad.replay_init(c, lad.ReplayBuffers(), 0)


def test_init_rejects_missing_or_misaligned_buffers(lad):
    c = lad.ReplayConfig(2, 4, 1, 64, 128, 16, lad.BF16, lad.NONE, 0)
    with pytest.raises(lad.ReplayError, match="status 1"):
        lad.replay_init(c, lad.ReplayBuffers(), 0)                 # all NULL
    bufs = lad.ReplayBuffers(*([0x1000] * 12))
    bufs.ring_v = 0x1008                                            # misaligned
    with pytest.raises(lad.ReplayError, match="status 1"):
        lad.replay_init(c, bufs, 0)


def test_calls_validate_before_touching_the_device(lad):
    c = lad.ReplayConfig(2, 4, 1, 64, 128, 16, lad.BF16, lad.NONE, 0)
    # NULL handle / pointers
    for fn, args in [(lad.lib.replay_decode, (None, 0x1000, None)),
                     (lad.lib.replay_verify, (None, 2, 0x1000, None)),
                     (lad.lib.replay_flush, (None, 1, None)),
                     (lad.lib.replay_rollback, (None, 0x1000, None)),
                     (lad.lib.replay_load_checkpoint, (None, 0x1000, None)),
                     (lad.lib.replay_append, (None, 1, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None)),
                     (lad.lib.replay_step, (None, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 16, None)),
                     (lad.lib.replay_step_static, (None, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 16, None)),
                     (lad.lib.replay_set_flush_skipping, (None, 0, None)),
                     (lad.lib.replay_set_flush_skipping, (None, 1, None))]:
        assert fn(*args) == 1
    # eager step: misaligned state pointer, unsupported shape
    assert lad.lib.replay_eager_step(ctypes.byref(c), 0x1004, 0x1000, 0x1000, 0x1000, 0x1000,
                                     0x1000, 0x1000, 0x1000, None) == 1
    bad = lad.ReplayConfig(2, 4, 1, 32, 128, 16, lad.BF16, lad.NONE, 0)
    assert lad.lib.replay_eager_step(ctypes.byref(bad), 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                                     0x1000, 0x1000, 0x1000, None) == 2
    # stream probe: bad mode, size not a multiple of 16
    assert lad.lib.replay_stream_probe(3, 0x1000, 0x2000, 64, None) == 1
    assert lad.lib.replay_stream_probe(0, 0x1000, 0x2000, 65, None) == 1
