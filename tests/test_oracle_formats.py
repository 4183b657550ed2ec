"""Pins of the oracle's number formats: bfloat16 decode, E4M3 encode/decode, MX block quantisation.

Pinned against the OFP8 table values (golden file), brute-force nearest-code search over the whole
E4M3 grid, exact round trips of representable blocks, and the binade the MX scale rule must put
each block's largest element in.
"""
import os

import numpy as np
import pytest

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_anchor_values.txt")


def _anchors():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


def test_bf16_decode_closed_forms():
    u = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x4B80], np.uint16)
    v = F.bf16_to_f64(u)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 2.0 ** -133  # smallest subnormal: 2**-126 * 2**-7
    assert v[3] == (2 - 2 ** -7) * 2.0 ** 127
    assert v[4] == 0.0 and np.signbit(v[4])
    assert v[5] == 2.0 ** 24


def test_e4m3_decode_matches_ofp8_table():
    for code, val in _anchors():
        got = F.e4m3_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_grid_shape():
    codes = np.arange(256, dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    assert np.isnan(vals).sum() == 2  # S.1111.111 only
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E strictly increasing
    assert pos[-1] == 448.0
    assert np.array_equal(vals[0x80:0xFF], -pos)


def test_e4m3_encode_decode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def _brute_force_encode(y):
    """Nearest E4M3 magnitude by exhaustive search; ties to the even code; clamp at 448."""
    grid = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    a = np.abs(y)[:, None]
    d = np.abs(a - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the code whose mantissa LSB is 0
    even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(np.abs(y) >= 448.0, 0x7E, pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def test_e4m3_encode_vs_brute_force_all_bf16_patterns():
    # every finite bfloat16 value, as is
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(u)
    v = v[np.isfinite(v)]
    assert np.array_equal(F.e4m3_encode(v), _brute_force_encode(v))


def test_e4m3_encode_vs_brute_force_dense_band():
    # every bfloat16 mantissa at every binade that can round to a non-zero E4M3 value, plus exact
    # midpoints between neighbouring codes (the ties)
    man = np.arange(128)
    vals = [(1 + man / 128.0) * 2.0 ** e for e in range(-12, 10)]
    grid = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    v = np.concatenate(vals + [mids, grid, [464.0, 480.0, 511.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    v = np.concatenate([v, -v])
    assert np.array_equal(F.e4m3_encode(v), _brute_force_encode(v))
    # a tie between 0x07 (7 * 2**-9) and 0x08 (8 * 2**-9) goes to the even code 0x08
    assert F.e4m3_encode(np.array([7.5 * 2.0 ** -9]))[0] == 0x08


def test_mx_zero_block_and_negative_zero():
    v = np.zeros((2, 32))
    v[1, 5] = -0.0
    q, s = F.mx_quantize(v)
    assert s.tolist() == [[0], [0]]
    assert q[1, 5] == 0x80 and np.count_nonzero(q) == 1


def test_mx_scale_puts_block_max_in_top_binade(rng):
    # floor(log2 amax) - 8: the block's largest element lands in [256, 512) before rounding, i.e.
    # on codes 0x78..0x7E after rounding and saturation
    for scale in [1e-30, 1e-6, 0.01, 1.0, 3.0, 1e5, 1e30]:
        v = rng.standard_normal((64, 32)) * scale
        q, s = F.mx_quantize(v)
        top = np.abs(F.e4m3_decode(q)).max(axis=1)
        assert np.all((top >= 256) & (top <= 448))
        amax = np.abs(v).max(axis=1)
        sv = s[:, 0].astype(np.int64) - 127
        assert np.all((amax >= 2.0 ** (sv + 8)) & (amax < 2.0 ** (sv + 9)))


def test_mx_exact_roundtrip_of_representable_blocks(rng):
    grid = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for s in [-127, -60, -8, 0, 5, 100, 119]:
        c = rng.choice(grid, size=(16, 32)) * rng.choice([-1.0, 1.0], size=(16, 32))
        c[:, 7] = rng.choice(grid[0x78:0x7F], size=16)  # amax in the top binade fixes the scale
        v = c * 2.0 ** s
        q, sc = F.mx_quantize(v)
        assert np.all(sc == s + 127)
        assert np.array_equal(F.mx_dequantize(q, sc), v)


def test_mx_saturation_band():
    v = np.zeros(32)
    v[0] = 500.0  # scale 2**0, 500 in [448, 512) saturates
    v[1] = 1.0
    q, s = F.mx_quantize(v)
    assert s[0] == 127 and q[0] == 0x7E and q[1] == 0x38


def test_mx_error_bound_and_axis(rng):
    v = rng.standard_normal((32, 96))
    deq = F.mx_roundtrip(v, axis=1)
    q, s = F.mx_quantize(v, axis=1)
    assert q.shape == v.shape and s.shape == (32, 3)
    sc = np.repeat(2.0 ** (s.astype(np.int64) - 127), 32, axis=1)
    y = np.abs(v) / sc
    # spacing of the E4M3 grid at |y|: 2**-9 below 2**-6, else 2**(floor(log2|y|) - 3)
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    spacing = 2.0 ** (e - 3)
    inside = y < 448.0
    assert np.all(np.abs(deq - v)[inside] <= (0.5 * spacing * sc)[inside])
    # the floor-based scale leaves [448, 512) * 2**s to saturation at 448 * 2**s
    assert np.all(deq[~inside] == np.sign(v[~inside]) * 448.0 * sc[~inside])
    assert (~inside).any()
    # quantising along axis 0 of the transpose gives the same numbers
    assert np.array_equal(F.mx_roundtrip(v.T, axis=0), deq.T)
    with pytest.raises(ValueError):
        F.mx_quantize(np.zeros((2, 33)))


def test_mx_roundtrip_equals_table_decode_of_quantize(rng):
    """The C round trip (in-place blocks, code values from the bit fields) equals decoding the
    codes mx_quantize gives through the OFP8-pinned value table, bit for bit, on every axis,
    including zeros of both signs, saturation, subnormal E4M3 results and extreme scales."""
    for shape, axis in [((64, 96), 0), ((64, 96), 1), ((6, 64, 40), 1), ((32,), 0),
                        ((5, 3, 64), -1), ((2, 32, 3, 5), 1)]:
        v = rng.standard_normal(shape) * np.exp2(rng.integers(-150, 128, size=shape))
        v.flat[::7] = 0.0
        v.flat[::11] *= -0.0
        v.flat[::13] = 460.0 * np.exp2(rng.integers(-20, 20))
        got = F.mx_roundtrip(v, axis)
        q, s = F.mx_quantize(v, axis)
        want = F.mx_dequantize(q, s, axis)
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), (shape, axis)
