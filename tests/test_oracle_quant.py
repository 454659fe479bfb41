"""The oracle's storage quantisers against torch's CPU float conversions and
the formats' own definitions (no GPU).

bf16: round to nearest even -- torch's float32 -> bfloat16 cast is the
library routine it must equal everywhere (NaN payloads aside).
e4m3fn: torch's float8_e4m3fn gives the OCP E4M3 table and round-to-nearest-
even conversion inside the finite range; beyond +-464 torch gives NaN while
the copy saturates to +-448 (the largest finite value), so those are pinned
by the format's closed form instead.
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _interesting_f32(rng, n):
    # random bit patterns over the whole range, plus exact bf16 midpoints (ties)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    mids = (rng.integers(0, 2 ** 16, size=n // 4, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 3.3895313892515355e38,
                         np.float32(3.4028235e38), np.float32(-3.4028235e38), 1e-45, -1e-45,
                         1.17549435e-38], dtype=np.float32)
    return np.concatenate([x, mids.view(np.float32), specials])


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(11)
    x = _interesting_f32(rng, 1 << 18)
    mine = oracle.bf16_encode(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.bf16_decode(mine[nan])))


def test_bf16_decode_matches_torch():
    codes = np.arange(1 << 16, dtype=np.uint16)
    mine = oracle.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok].view(np.uint32), ref[ok].view(np.uint32))


def test_e4m3_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok].view(np.uint32), ref[ok].view(np.uint32))
    # closed forms of the format
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(12)
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[1:] + vals[:-1]) / 2                    # exact ties
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rand = np.concatenate([rng.uniform(-464, 464, 200000), rng.standard_normal(100000) * 1e-2,
                           rng.standard_normal(100000) * 1e-3])
    x = np.concatenate([vals, -vals, mids, -mids, near, -near, rand, [464.0, -464.0, 0.0, -0.0]]).astype(np.float32)
    mine = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_saturates_and_nan():
    x = np.array([464.0001, 465, 500, 1e6, np.inf, 3.4e38], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(x) == 0x7E)
    assert np.all(oracle.e4m3_encode(-x) == 0xFE)
    nan = oracle.e4m3_encode(np.array([np.nan], dtype=np.float32))
    assert (nan[0] & 0x7F) == 0x7F


def test_e4m3_ties_go_to_even_code():
    # 1 + 1/16 lies halfway between 1 (code 0x38, even) and 1.125 (0x39)
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10], dtype=np.float32)
    assert list(oracle.e4m3_encode(x)) == [0x38, 0x3A, 0x00, 0x02]


def test_quant_heads_scale_and_extremes():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 2, 8, 16)).astype(np.float32)
    x[1, 1] = 0.0
    codes, scale = oracle.quant_heads_e4m3(x)
    amax = np.max(np.abs(x), axis=(-1, -2))
    expect = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    assert np.array_equal(scale, expect)
    assert np.all(codes[1, 1] == 0)
    # the element of largest magnitude lands on +-448 (code 0x7E / 0xFE)
    for i in range(3):
        for j in range(2):
            if amax[i, j] == 0:
                continue
            idx = np.unravel_index(np.argmax(np.abs(x[i, j])), x[i, j].shape)
            assert codes[i, j][idx] & 0x7F == 0x7E
    # every code equals the element-wise conversion of x / scale (float32 divide)
    r = (x / scale[..., None, None]).astype(np.float32)
    assert np.array_equal(codes, oracle.e4m3_encode(r))
    # dequantised values are within half a code step of the inputs
    deq = oracle.e4m3_decode(codes) * scale[..., None, None]
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + scale[..., None, None] * 2.0 ** -10)


# ---- E2M1 (FP4) and MX block scaling -----------------------------------------
# The OCP MX specification's table of E2M1 magnitudes (codes 0..7); codes
# 8..15 are their negatives.  The oracle's decoder is built from the bit
# fields, so this table pins it from outside.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_is_the_published_table():
    vals = oracle.core.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert vals[:8].tolist() == E2M1_TABLE
    assert vals[8:].tolist() == [-v for v in E2M1_TABLE]
    assert np.signbit(vals[8])


def _nearest_even(x):
    """Brute force: nearest table magnitude, ties to the even code, saturating."""
    mags = np.array(E2M1_TABLE)
    out = []
    for v in x:
        a = min(abs(v), 6.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        out.append(c | (8 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(11)
    grid = np.arange(-800, 801) / 100.0                      # every 0.01 in [-8, 8], ties included
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0])
    x = np.concatenate([grid, mids, rng.uniform(-10, 10, 2000), [100.0, -1e30, 6.0000001, -0.0]])
    assert np.array_equal(oracle.core.e2m1_encode(x), _nearest_even(x))


def test_mx_block_scale_closed_forms():
    rng = np.random.default_rng(12)
    # a block whose largest magnitude lies in [4 * 2^k, 8 * 2^k) gets X = 2^k (E8M0 byte 127 + k)
    for k in (-20, -3, 0, 1, 7, 30):
        blk = rng.uniform(-1, 1, (1, 32)).astype(np.float32) * np.float32(2.0 ** k)
        blk[0, 5] = np.float32(rng.uniform(4, 8) * 2.0 ** k)
        blk = np.clip(blk, -blk[0, 5], blk[0, 5])
        packed, scale = oracle.core.quant_blocks_mxfp4(blk)
        assert scale.ravel().tolist() == [127 + k]
        assert ((packed.ravel()[2] >> 4) & 0x7) in (6, 7)     # the largest element (index 5, high nibble of byte 2)
    # exactly representable values come back exactly, packing order low nibble first
    codes = rng.integers(0, 16, 32).astype(np.uint8)
    codes[3] = 7                                              # amax = 6 X
    X = 2.0 ** -5
    blk = (oracle.core.e2m1_decode(codes).astype(np.float64) * X).astype(np.float32).reshape(1, 32)
    packed, scale = oracle.core.quant_blocks_mxfp4(blk)
    assert scale.ravel().tolist() == [127 - 5]
    assert np.array_equal(packed.ravel() & 0xF, codes[0::2])
    assert np.array_equal(packed.ravel() >> 4, codes[1::2])
    back = oracle.core.dequant_blocks_mxfp4(packed, scale, blk.shape)
    assert np.array_equal(np.abs(back), np.abs(blk))
    # an all-zero block: scale 2^-127, all codes zero
    packed, scale = oracle.core.quant_blocks_mxfp4(np.zeros((2, 16), np.float32))
    assert scale.ravel().tolist() == [0] and not packed.any()


def test_mx_block_error_bounds():
    """Round to nearest: |deq - x| <= X/4 below X (spacing X/2) and <= X at
    the top (spacing 2X between 4X and 6X); saturated values sit at 6X <= amax."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((64, 4, 32)) * np.exp(rng.uniform(-8, 8, (64, 1, 1)))).astype(np.float32)
    packed, scale = oracle.core.quant_blocks_mxfp4(x)
    back = oracle.core.dequant_blocks_mxfp4(packed, scale, x.shape).astype(np.float64)
    X = np.exp2(scale.astype(np.float64) - 127).reshape(64, 4, 1)
    xd = x.astype(np.float64)
    err = np.abs(back - xd)
    small = np.abs(xd) < X
    assert np.all(err[small] <= X.repeat(32, -1)[small] / 4)
    assert np.all(err <= np.maximum(X, np.abs(xd) - 6 * X) + 0 * err)
    amax = np.abs(xd).max(-1, keepdims=True)
    assert np.all((amax >= 4 * X) & (amax < 8 * X))
