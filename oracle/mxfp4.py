"""MXFP4 (E2M1 elements + E8M0 shared scale per 32 values), float64 reference.

The KroQuant page (§03) quantizes to an MXFP4 format it calls "MXFP4e2"; the element
and scale rules are those of the OCP Microscaling Formats (MX) v1.0 spec:

* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6; no Inf/NaN.  Conversion rounds to nearest, ties to
  even, and saturates at 6.
* E8M0 shared scale: an unbiased power-of-two exponent e stored as e + 127.  The
  spec's rule picks e = floor(log2(amax)) - emax_elem with emax_elem = 2 for E2M1,
  so the block maximum lands in [4, 8) after scaling and values in (6, 8) saturate.

Readings taken where the pages are silent: the code of a value is
sign_bit*8 | magnitude_index, with sign_bit = (value < 0), so an exact zero is
0x0 and a negative value that rounds to zero is 0x8; an all-zero block gets
e = -127 (byte 0x00); element 2i sits in the low nibble of byte i.
"""

import math

import numpy as np

# Magnitudes of the eight non-negative E2M1 codes, in code order (index = code & 7).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_EMAX = 2          # exponent of the largest normal E2M1 magnitude (6 = 1.5 * 2^2)
E8M0_BIAS = 127
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127
BLOCK = 32


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (uint8 array, values 0..15)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def e2m1_encode(s):
    """Round float64 values to E2M1 codes: nearest magnitude, ties to the even index.

    Written as an explicit nearest-neighbour search over the eight magnitudes, after
    saturating magnitudes above 6 to 6 (the spec's saturating conversion; without the
    clamp, float64 distances to a huge value would all round to the same number).
    """
    s = np.asarray(s, dtype=np.float64)
    a = np.minimum(np.abs(s), E2M1_MAGNITUDES[-1])
    dist = np.abs(a[..., None] - E2M1_MAGNITUDES)            # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    is_best = dist == best
    # Among equally near magnitudes (a tie can involve at most two), keep the even index.
    idx = np.arange(8)
    even_best = is_best & (idx % 2 == 0)
    choice = np.where(even_best.any(axis=-1), np.argmax(even_best, axis=-1), np.argmax(is_best, axis=-1))
    sign = (s < 0).astype(np.uint8)
    return (sign * 8 + choice).astype(np.uint8)


def e8m0_exponent(amax):
    """Shared exponent e of a block from its largest magnitude (OCP MX rule).

    floor(log2 a) is taken from frexp (a = m * 2**x, m in [0.5, 1)), never from a
    floating-point log2.  e = floor(log2 a) - 2, clamped to [-127, 127]; a = 0 gives -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    out = np.empty(amax.shape, dtype=np.int64)
    flat_a = amax.reshape(-1)
    flat_o = out.reshape(-1)
    for i, a in enumerate(flat_a):
        if a == 0.0:
            flat_o[i] = E8M0_MIN_EXP
        else:
            _, x = math.frexp(float(a))
            flat_o[i] = min(max((x - 1) - E2M1_EMAX, E8M0_MIN_EXP), E8M0_MAX_EXP)
    return out


def quantize_blocks(y):
    """MXFP4-quantize float64 rows along their last axis in blocks of 32.

    Returns (codes uint8 [..., K] one code per element, scale bytes uint8 [..., K/32],
    exponents int64 [..., K/32]).
    """
    y = np.asarray(y, dtype=np.float64)
    K = y.shape[-1]
    assert K % BLOCK == 0
    blocks = y.reshape(y.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    e = e8m0_exponent(amax)
    scaled = blocks * np.ldexp(1.0, -e)[..., None]          # exact: power-of-two scaling
    codes = e2m1_encode(scaled).reshape(y.shape)
    return codes, (e + E8M0_BIAS).astype(np.uint8), e


def dequantize(codes, scale_bytes):
    """Float64 values of unpacked codes [..., K] with their E8M0 bytes [..., K/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    e = scale_bytes.astype(np.int64) - E8M0_BIAS
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (K // BLOCK, BLOCK))
    return (vals * np.ldexp(1.0, e)[..., None]).reshape(codes.shape)


def pack_nibbles(codes):
    """Two codes per byte: element 2i in bits 0-3, element 2i+1 in bits 4-7."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out
