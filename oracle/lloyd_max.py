"""Lloyd-Max scalar quantizers for N(0, 1) and the per-token / per-group quantizers
that use them, float64.

OrbitQuant page, §03: after the RPBH rotation every coordinate is close to Gaussian,
so one fixed Lloyd-Max codebook serves all timesteps and layers.  CentriQ page,
arXiv abstract: the per-token scale then follows in closed form without data.

Readings taken where the pages are silent:
* the codebook is the symmetric fixed point of Lloyd's iteration for N(0, 1)
  (levels are conditional means of their cells, thresholds are midpoints);
* the per-token scale is the RMS of the rotated token, s_t = sqrt(mean(y_t^2)),
  the Gaussian-matched scale for an N(0, 1) codebook; it is stored as float32 and
  the codes are decided against the stored value;
* codes are sign-magnitude: sign bit = (value < 0), magnitude index counts the
  positive thresholds strictly below |value / s| (a value on a threshold goes to the
  smaller magnitude); a zero scale gives all-zero codes;
* 2-bit weights (W2): 4-level codebook, one fp16 scale per 32 weights along K
  (s_g = fp16(RMS of the group)), codes decided against the stored fp16 scale,
  packed four per byte with the lowest k in the lowest bits.
"""

import numpy as np
from scipy import special


def _phi(t):
    return np.exp(-0.5 * t * t) / np.sqrt(2.0 * np.pi)


def _mass(a, b):
    """P(a < Z < b) for Z ~ N(0, 1), accurate in the upper tail (a >= 0)."""
    return special.ndtr(-a) - special.ndtr(-b)


def lloyd_max_levels(n_levels, tol=1e-15, max_iter=200000):
    """Positive levels (ascending) of the symmetric n-level Lloyd-Max quantizer for N(0, 1)."""
    assert n_levels % 2 == 0
    half = n_levels // 2
    # start from equal-probability cells on the positive half line
    qs = special.ndtri(0.5 + 0.5 * (np.arange(half) + 0.5) / half)
    levels = np.asarray(qs, dtype=np.float64)
    for _ in range(max_iter):
        thr = np.concatenate(([0.0], 0.5 * (levels[:-1] + levels[1:]), [np.inf]))
        lo, hi = thr[:-1], thr[1:]
        phi_hi = np.where(np.isinf(hi), 0.0, _phi(np.where(np.isinf(hi), 0.0, hi)))
        new = (_phi(lo) - phi_hi) / _mass(lo, hi)          # E[Z | lo < Z < hi]
        if np.max(np.abs(new - levels)) <= tol:
            levels = new
            break
        levels = new
    return levels


def thresholds(levels):
    """Positive decision thresholds between consecutive positive levels."""
    return 0.5 * (levels[:-1] + levels[1:])


def fixed_point_residual(levels):
    thr = np.concatenate(([0.0], thresholds(levels), [np.inf]))
    lo, hi = thr[:-1], thr[1:]
    phi_hi = np.where(np.isinf(hi), 0.0, _phi(np.where(np.isinf(hi), 0.0, hi)))
    cm = (_phi(lo) - phi_hi) / _mass(lo, hi)
    return float(np.max(np.abs(cm - levels)))


def mse(levels):
    """Mean squared error of the symmetric quantizer on N(0, 1) (numerical integration)."""
    from scipy import integrate
    thr = np.concatenate(([0.0], thresholds(levels), [np.inf]))
    total = 0.0
    for c, lo, hi in zip(levels, thr[:-1], thr[1:]):
        val, _ = integrate.quad(lambda z, c=c: (z - c) ** 2 * _phi(z), lo, hi, epsabs=1e-14)
        total += 2.0 * val
    return total


LEVELS16 = lloyd_max_levels(16)
LEVELS4 = lloyd_max_levels(4)


def sign_magnitude_encode(v, thr):
    """Code of each value v (already divided by its scale): sign*(2^bits/2) | index."""
    v = np.asarray(v, dtype=np.float64)
    idx = (np.abs(v)[..., None] > thr).sum(axis=-1)
    half = len(thr) + 1
    return ((v < 0).astype(np.int64) * half + idx).astype(np.uint8)


def sign_magnitude_decode(codes, levels):
    codes = np.asarray(codes, dtype=np.int64)
    half = len(levels)
    mag = levels[codes % half]
    return np.where(codes >= half, -mag, mag)


def lm4_token_quantize(y):
    """Per-token Lloyd-Max 4-bit quantization of rotated rows y [M, K].

    Returns (codes uint8 [M, K], scale float32 [M]).
    """
    y = np.asarray(y, dtype=np.float64)
    s_exact = np.sqrt(np.mean(y * y, axis=1))
    s = s_exact.astype(np.float32)
    s64 = s.astype(np.float64)
    thr = thresholds(LEVELS16)
    codes = np.zeros(y.shape, dtype=np.uint8)
    nz = s64 > 0
    codes[nz] = sign_magnitude_encode(y[nz] / s64[nz, None], thr)
    return codes, s


def lm4_dequantize(codes, s):
    return sign_magnitude_decode(codes, LEVELS16) * np.asarray(s, dtype=np.float64)[:, None]


def w2_group_quantize(wt):
    """2-bit Lloyd-Max quantization of rows wt [N, K] in groups of 32 along K.

    Returns (codes uint8 [N, K], group scales float16 [N, K/32]).
    """
    wt = np.asarray(wt, dtype=np.float64)
    N, K = wt.shape
    g = wt.reshape(N, K // 32, 32)
    s = np.sqrt(np.mean(g * g, axis=2)).astype(np.float16)
    s64 = s.astype(np.float64)
    thr = thresholds(LEVELS4)
    codes = np.zeros(g.shape, dtype=np.uint8)
    nz = s64 > 0
    codes[nz] = sign_magnitude_encode(g[nz] / s64[nz][:, None], thr)
    return codes.reshape(N, K), s


def w2_dequantize(codes, s):
    N, K = codes.shape
    vals = sign_magnitude_decode(codes, LEVELS4).reshape(N, K // 32, 32)
    return (vals * np.asarray(s, dtype=np.float64)[..., None]).reshape(N, K)


def pack_2bit(codes):
    """Four 2-bit codes per byte, element 4i in bits 0-1 ... element 4i+3 in bits 6-7."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def unpack_2bit(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 4,), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (p >> (2 * j)) & 3
    return out
