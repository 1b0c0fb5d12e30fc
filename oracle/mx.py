"""MXFP8 (OCP Microscaling v1.0, E4M3 elements, E8M0 block scale) in fp64. TEST INFRASTRUCTURE ONLY.

The Notes ("The production details") say only that the layer supports MXFP8, with activation
quantisation fused into dispatch, the grouped GEMMs and the gated activation. The encoding is
the published OCP MX v1.0 one:

* a block is 32 consecutive elements along the contraction dimension;
* the block scale is X = 2^(floor(log2(amax)) - emax_elem) with emax_elem = 8 for E4M3, stored
  as an E8M0 byte (biased exponent, bias 127), clamped to the representable range [-127, 127];
* each element is v / X rounded to nearest-even on the E4M3 grid (4 exponent bits, bias 7,
  3 mantissa bits, subnormals below 2^-6, no infinities), saturating at +-448;
* a block whose amax is 0 gets the scale byte 127 and all-zero elements.
"""
from __future__ import annotations

import numpy as np

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal (448 = 1.75 * 2^8)
E4M3_EMIN = -6         # exponent of the smallest normal
E4M3_MBITS = 3


def _floor_log2(a):
    """floor(log2(a)) for a > 0, exact (frexp gives a = m * 2^ex with m in [0.5, 1))."""
    _, ex = np.frexp(a)
    return ex.astype(np.int64) - 1


def e4m3_round(y):
    """Nearest E4M3 value (ties to even), saturating at +-448. fp64 in, fp64 out; sign kept."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    safe = np.where(a > 0, a, 1.0)
    e = np.maximum(_floor_log2(safe), E4M3_EMIN)
    quantum = np.ldexp(1.0, (e - E4M3_MBITS).astype(np.int32))
    r = np.round(a / quantum) * quantum          # np.round rounds halves to even
    r = np.where(a > 0, np.minimum(r, E4M3_MAX), 0.0)
    return np.copysign(r, y)


def e4m3_encode(r):
    """Bit pattern (uint8) of values already on the E4M3 grid (as from e4m3_round)."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.uint8)
    a = np.abs(r)
    safe = np.where(a > 0, a, 1.0)
    e = _floor_log2(safe)
    normal = (a >= 2.0 ** E4M3_EMIN)
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, np.ldexp(a, (-e).astype(np.int32)) * 8 - 8, a / 2.0 ** (E4M3_EMIN - 3))
    mant = np.where(a > 0, mant, 0)
    assert np.all(mant == np.round(mant)), 'value not on the E4M3 grid'
    return ((sign << 7) | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(b):
    """E4M3 byte -> fp64 value (0x7F / 0xFF, the NaN codes, decode to NaN)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ef = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(ef == 0, m / 8.0 * 2.0 ** E4M3_EMIN,
                   (1.0 + m / 8.0) * np.ldexp(1.0, (ef - 7).astype(np.int32)))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def mx_quantize(v):
    """Quantise v [..., n] along its last axis (n a multiple of 32).

    Returns (q uint8 [..., n] E4M3 codes, scale uint8 [..., n/32] E8M0 codes).
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    assert n % MX_BLOCK == 0
    blk = v.reshape(v.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    safe = np.where(amax > 0, amax, 1.0)
    shared = np.clip(_floor_log2(safe) - E4M3_EMAX, -127, 127)
    shared = np.where(amax > 0, shared, 0)
    scaled = blk / np.ldexp(1.0, shared.astype(np.int32))[..., None]
    q = e4m3_encode(e4m3_round(scaled)).reshape(v.shape)
    return q, (shared + 127).astype(np.uint8)


def mx_dequantize(q, scale):
    """Inverse of mx_quantize: element value times 2^(scale - 127)."""
    q = np.asarray(q, dtype=np.uint8)
    n = q.shape[-1]
    vals = e4m3_decode(q).reshape(q.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    sc = np.ldexp(1.0, np.asarray(scale, dtype=np.int64).astype(np.int32) - 127)
    return (vals * sc[..., None]).reshape(q.shape)


def mx_roundtrip(v):
    """Quantise then dequantise (the value an MXFP8 operand stands for)."""
    return mx_dequantize(*mx_quantize(v))
