"""Number formats of the oracle: bfloat16 decode, OCP E4M3 and the MX block scale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E4M3 follows the OCP 8-bit Floating Point specification (OFP8) v1.0: one sign bit, four exponent
bits with bias 7, three mantissa bits; exponent field 0 holds subnormals m * 2**-9; there is no
infinity, S.1111.111 is NaN, so the largest finite magnitude is S.1111.110 = 1.75 * 2**8 = 448.

An MX block (OCP Microscaling Formats v1.0, MXFP8 E4M3) is 32 consecutive elements that share one
E8M0 scale, a power of two 2**s stored as the byte s + 127 (255 is NaN). The spec's conversion sets
s = floor(log2(amax)) - emax_elem with emax_elem = 8 for E4M3, divides every element by 2**s and
rounds it to E4M3, clamping to the largest normal.

Readings where the pages (and the spec) leave a choice open:
  * amax == 0: s = -127, scale byte 0x00, elements encode as zeros.
  * s is clamped to [-127, 127].
  * The sign of zero is kept: -0.0 encodes as 0x80.
  * Magnitudes >= 448 after scaling saturate to 448 (0x7E / 0xFE); NaN (0x7F) is never produced.
  * Rounding is to nearest, ties to even mantissa (the default IEEE rounding the spec assumes).
"""
from __future__ import annotations

import numpy as np

from . import _native

MX_BLOCK = 32
E4M3_EMAX = 8  # exponent of the largest normal, 448 = 1.75 * 2**8
E4M3_MAX = 448.0
E8M0_BIAS = 127


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): a bfloat16 is the top half of a float32."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """E4M3 byte -> float64 value, straight from the bit-field definition (NaN for S.1111.111)."""
    c = np.asarray(c, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    sub = man * 2.0 ** -9  # (man / 8) * 2**(1 - 7)
    nor = (1.0 + man / 8.0) * np.exp2((ex - 7).astype(np.float64))
    val = sign * np.where(ex == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


_E4M3_VALUES = _e4m3_value(np.arange(256))  # the value of every byte


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 byte -> float64 value (the bit-field definition, evaluated once for all 256 bytes)."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float64 -> E4M3 byte: round to nearest even, saturate at 448, keep the sign of zero.

    Normal range: with |y| = f * 2**e, 1 <= f < 2, the mantissa code is round(|y| * 2**(3 - e)) - 8;
    a rounding up to 16 carries into the exponent. Below 2**-6 the grid is n * 2**-9, n = 0..8,
    and n = 8 is the smallest normal (code 0x08). The loop over elements is in mx_codec.c.
    """
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    _native.lib().oracle_e4m3_encode(y.ctypes.data, out.ctypes.data, y.size)
    return out


def mx_quantize(v: np.ndarray, axis: int = -1):
    """MX-quantise along ``axis`` in blocks of 32 consecutive elements.

    Returns (codes uint8, same shape as v; scales uint8, shape with that axis divided by 32).
    The length along ``axis`` must be a multiple of 32.

    Per block: s = floor(log2 amax) - 8 (amax > 0), clamped to [-127, 127], else -127; every
    element is divided by 2**s and encoded with e4m3_encode. The loop over blocks is in
    mx_codec.c.
    """
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    n = v.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("MX blocks need a length that is a multiple of 32")
    rows = np.ascontiguousarray(v).reshape(-1, n)
    codes = np.empty(rows.shape, dtype=np.uint8)
    scales = np.empty((rows.shape[0], n // MX_BLOCK), dtype=np.uint8)
    _native.lib().oracle_mx_quantize_rows(rows.ctypes.data, rows.shape[0], n, codes.ctypes.data,
                                          scales.ctypes.data)
    codes = codes.reshape(v.shape)
    scales = scales.reshape(v.shape[:-1] + (n // MX_BLOCK,))
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, axis: int = -1) -> np.ndarray:
    """Inverse map of ``mx_quantize``: 2**s * decode(code), float64."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1).astype(np.int64) - E8M0_BIAS
    vals = e4m3_decode(c)
    vals = vals.reshape(vals.shape[:-1] + (vals.shape[-1] // MX_BLOCK, MX_BLOCK))
    out = (vals * np.exp2(s.astype(np.float64))[..., None]).reshape(c.shape)
    return np.moveaxis(out, -1, axis)


def mx_roundtrip(v: np.ndarray, axis: int = -1) -> np.ndarray:
    """The value each element of v takes after MX quantisation along ``axis``: 2**s times the value
    of its E4M3 code, as mx_dequantize(mx_quantize(v, axis), axis) gives.

    The loop is in mx_codec.c and walks the blocks in place (no transposed copy), with the same
    scale rule and encoder as mx_quantize and the code's value from its bit fields."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    ax = axis % v.ndim
    L = v.shape[ax]
    if L % MX_BLOCK:
        raise ValueError("MX blocks need a length that is a multiple of 32")
    outer = int(np.prod(v.shape[:ax], dtype=np.int64))
    inner = int(np.prod(v.shape[ax + 1:], dtype=np.int64))
    out = np.empty_like(v)
    amax = np.empty(max(inner, 1), dtype=np.float64)
    _native.lib().oracle_mx_roundtrip_axis(v.ctypes.data, out.ctypes.data, outer, L, inner,
                                           amax.ctypes.data)
    return out
