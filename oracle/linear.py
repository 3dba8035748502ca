"""The 4-bit linear with its full-precision branches, float64.

Y = Xq Wq'^T + (X L1^T) L2^T + mu wbar^T

* Xq Wq'^T: the 4-bit product in the transformed basis, (XP)(P^-1 W)
  (KroQuant §01; OrbitQuant §03 W' = R^-1 W), computed by dequantizing both
  operands to float64 and calling np.matmul.  Every E2M1 x E2M1 x 2^e product is
  exact in float64, so this equals the per-block scaled-sum form exactly up to the
  order of the float64 additions.
* (X L1^T) L2^T: the 16-bit low-rank branch of SVDQuant (explainer §3), fed by the
  original (untransformed, uncentred) fp16 activations.
* mu wbar^T: CentriQ's rank-1 mean restore (arXiv abstract).

Weight operands use the [out][in] layout: W'^T codes [N][K/2], L1 [r][K], L2 [N][r].
No bias.  The result is returned in float64; the GPU's fp16 output is compared to it.
"""

import numpy as np

from . import lloyd_max, mxfp4


def _rows(a, rows):
    return a if rows is None else a[rows]


def dequant_mxfp4(codes_packed, scale_bytes, rows=None):
    c = mxfp4.unpack_nibbles(_rows(codes_packed, rows))
    return mxfp4.dequantize(c, _rows(scale_bytes, rows))


def dequant_lm4(codes_packed, s, rows=None):
    c = mxfp4.unpack_nibbles(_rows(codes_packed, rows))
    return lloyd_max.lm4_dequantize(c, _rows(s, rows))


def dequant_w2(codes_packed, s, rows=None):
    c = lloyd_max.unpack_2bit(_rows(codes_packed, rows))
    return lloyd_max.w2_dequantize(c, _rows(s, rows))


def lowrank_term(X_f16, L1_rk, L2_nr, rows=None, cols=None):
    X = np.asarray(_rows(X_f16, rows), dtype=np.float64)
    T = X @ np.asarray(L1_rk, dtype=np.float64).T                  # [m, r]
    L2 = np.asarray(_rows(L2_nr, cols), dtype=np.float64)          # [n, r]
    return T @ L2.T


def linear(xd, wd, X_f16=None, L1_rk=None, L2_nr=None, mu=None, wbar=None,
           rows=None, cols=None, chunk=1024):
    """Y[rows][cols] from dequantized float64 operands xd [M, K], wd [N, K] (already sliced
    to rows/cols by the caller) plus the optional branches (sliced here)."""
    M = xd.shape[0]
    Y = np.empty((M, wd.shape[0]), dtype=np.float64)
    for s in range(0, M, chunk):
        Y[s:s + chunk] = np.matmul(xd[s:s + chunk], wd.T)
    if L1_rk is not None:
        Y += lowrank_term(X_f16, L1_rk, L2_nr, rows, cols)
    if mu is not None:
        m = np.asarray(_rows(mu, rows), dtype=np.float64)
        w = np.asarray(_rows(wbar, cols), dtype=np.float64)
        Y += m[:, None] * w[None, :]
    return Y


def w4a4_linear(xcodes, xscales, wcodes, wscales, X_f16=None, L1_rk=None, L2_nr=None,
                mu=None, wbar=None, rows=None, cols=None):
    xd = dequant_mxfp4(xcodes, xscales, rows)
    wd = dequant_mxfp4(wcodes, wscales, cols)
    return linear(xd, wd, X_f16, L1_rk, L2_nr, mu, wbar, rows, cols)


def w2a4_linear(xcodes, xscales, wcodes, wscales, rows=None, cols=None):
    xd = dequant_lm4(xcodes, xscales, rows)
    wd = dequant_w2(wcodes, wscales, cols)
    return linear(xd, wd, rows=rows, cols=cols)


def rel_frobenius(y_test, y_ref):
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(y_test - y_ref) / np.linalg.norm(y_ref))
