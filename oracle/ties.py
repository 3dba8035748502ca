"""Classification of code mismatches between a float32 kernel and the float64 oracle.

Where floating point decides an integer (a 4-bit code, a shared exponent, an fp16
mean), a kernel that computes in float32 may decide differently from the exact
float64 value when that value lies within the kernel's forward error bound of a
decision boundary.  Such a mismatch is a *tie*: both answers are correct roundings
of values the two sides can legitimately hold.  Every other mismatch is an error.

Error bounds: for a sum of n products evaluated in float32 (any order, one rounding
per operation) the forward error is at most gamma_n * sum|terms| with
gamma_n = n u / (1 - n u), u = 2^-24 (Higham, Accuracy and Stability of Numerical
Algorithms, §3.1).  Callers pass tau (per element, in unscaled units) computed with
a safety factor of 2 on top of that bound.

E2M1 decision boundaries on the scaled magnitude: 0.25, 0.75, 1.25, 1.75, 2.5, 3.5,
5, plus 0 for the sign of a value whose magnitude rounds to zero.  The shared
exponent changes at every power of two of the block maximum.
"""

import math

import numpy as np

from . import lloyd_max, mxfp4

U32 = 2.0 ** -24


def gamma_tau(n, abs_sum, safety=2.0):
    """tau = safety * gamma_n * abs_sum (elementwise)."""
    g = n * U32 / (1.0 - n * U32)
    return safety * g * np.asarray(abs_sum, dtype=np.float64)


def _near_power_of_two(a, tau):
    """True if some power of two lies within [a - tau, a + tau] (a > 0)."""
    if a <= 0.0:
        return tau > 0.0 and False
    lo, hi = a - tau, a + tau
    if lo <= 0.0:
        return True
    _, x = math.frexp(hi)
    p = math.ldexp(1.0, x - 1)          # largest power of two <= hi
    return p >= lo


def classify_mxfp4(gpu_codes, gpu_scale_bytes, y, tau, log_limit=50):
    """Compare MXFP4 codes/scales from a kernel with the exact transformed values y.

    gpu_codes: uint8 [M, K] unpacked codes; gpu_scale_bytes: uint8 [M, K/32];
    y: float64 [M, K] exact transformed values; tau: float64 [M, K] error bound.
    Returns a dict with counts, a tie log (row, block, k, value, boundary, tau) and the
    error list (non-tie mismatches).
    """
    M, K = y.shape
    nb = K // 32
    ref_codes, ref_bytes, ref_e = mxfp4.quantize_blocks(y)
    gpu_e = gpu_scale_bytes.astype(np.int64) - mxfp4.E8M0_BIAS
    yb = y.reshape(M, nb, 32)
    tb = tau.reshape(M, nb, 32)
    gc = gpu_codes.reshape(M, nb, 32)
    rc = ref_codes.reshape(M, nb, 32)
    report = dict(codes=M * K, blocks=M * nb, scale_mismatch=0, scale_ties=0, code_mismatch=0,
                  code_ties=0, errors=[], ties=[])

    bad_scale = np.argwhere(gpu_e != ref_e)
    for (m, b) in bad_scale:
        report["scale_mismatch"] += 1
        amax = float(np.abs(yb[m, b]).max())
        tmax = float(tb[m, b].max())
        if abs(int(gpu_e[m, b]) - int(ref_e[m, b])) == 1 and _near_power_of_two(amax, tmax):
            report["scale_ties"] += 1
            if len(report["ties"]) < log_limit:
                report["ties"].append(("scale", int(m), int(b), -1, amax, "2^k", tmax))
        else:
            report["errors"].append(("scale", int(m), int(b), int(gpu_e[m, b]), int(ref_e[m, b]), amax, tmax))

    # codes, judged against the exponent the kernel chose for the block (after a scale tie
    # the oracle re-derives the block with the kernel's exponent)
    scale = np.ldexp(1.0, -gpu_e)[..., None]
    s = yb * scale
    ts = tb * scale
    ref_at_gpu_e = mxfp4.e2m1_encode(s)
    mism = np.argwhere(gc != ref_at_gpu_e)
    report["code_mismatch"] = int(np.count_nonzero(gc != rc))
    for (m, b, k) in mism:
        v, t = float(s[m, b, k]), float(ts[m, b, k])
        lo = int(mxfp4.e2m1_encode(np.array(v - t)))
        hi = int(mxfp4.e2m1_encode(np.array(v + t)))
        g = int(gc[m, b, k])
        if lo != hi and g in (lo, hi):
            report["code_ties"] += 1
            if len(report["ties"]) < log_limit:
                report["ties"].append(("code", int(m), int(b), int(k), v, _nearest_boundary(v), t))
        else:
            report["errors"].append(("code", int(m), int(b), int(k), g, int(ref_at_gpu_e[m, b, k]), v, t))
    return report


_E2M1_BOUNDS = np.array([0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _nearest_boundary(v):
    a = abs(v)
    return float(_E2M1_BOUNDS[np.argmin(np.abs(_E2M1_BOUNDS - a))])


def classify_lm4(gpu_codes, gpu_s, y, tau, s_rel_tol, log_limit=50):
    """Compare per-token Lloyd-Max codes and scales with the exact rotated values y.

    gpu_s: float32 [M] kernel scales; s_rel_tol: relative error bound of the kernel's
    scale.  A code mismatch is a tie when the value, perturbed by the kernel's error
    bound on y and on s, can land on either side of a threshold.
    """
    M, K = y.shape
    ref_codes, ref_s = lloyd_max.lm4_token_quantize(y)
    thr = lloyd_max.thresholds(lloyd_max.LEVELS16)
    report = dict(codes=M * K, rows=M, scale_errors=0, code_mismatch=0, code_ties=0,
                  errors=[], ties=[])
    s_ref64 = np.sqrt(np.mean(y * y, axis=1))
    rel = np.abs(gpu_s.astype(np.float64) - s_ref64) / np.maximum(s_ref64, 1e-300)
    for m in np.argwhere(rel > s_rel_tol).reshape(-1):
        report["scale_errors"] += 1
        report["errors"].append(("scale", int(m), float(gpu_s[m]), float(s_ref64[m])))
    mism = np.argwhere(gpu_codes != ref_codes)
    report["code_mismatch"] = len(mism)
    for (m, k) in mism:
        s = float(ref_s[m])
        if s == 0.0:
            report["errors"].append(("code", int(m), -1, int(k), int(gpu_codes[m, k]), int(ref_codes[m, k])))
            continue
        v = float(y[m, k]) / s
        d = float(tau[m, k]) / s + abs(v) * (s_rel_tol + 2 * U32)
        lo = int(lloyd_max.sign_magnitude_encode(np.array(v - d), thr))
        hi = int(lloyd_max.sign_magnitude_encode(np.array(v + d), thr))
        g = int(gpu_codes[m, k])
        if lo != hi and g in (lo, hi):
            report["code_ties"] += 1
            if len(report["ties"]) < log_limit:
                report["ties"].append(("code", int(m), -1, int(k), v, "LM threshold", d))
        else:
            report["errors"].append(("code", int(m), -1, int(k), g, int(ref_codes[m, k]), v, d))
    return report


def mean_tie(x_row_f16, mu_gpu_f16, mu_ref_f16, n_terms):
    """True if the two fp16 means are adjacent roundings of a mean that lies within the
    float32 summation bound of the fp16 rounding midpoint between them."""
    x = np.asarray(x_row_f16, dtype=np.float64)
    exact = float(np.mean(x))
    a, b = float(mu_gpu_f16), float(mu_ref_f16)
    if a == b:
        return True
    nxt = np.nextafter(np.float16(min(a, b)), np.float16(np.inf))
    if float(nxt) != max(a, b):
        return False                       # not adjacent fp16 values
    mid = 0.5 * (a + b)
    bound = float(gamma_tau(n_terms, np.sum(np.abs(x)) / len(x)))
    return abs(exact - mid) <= bound
