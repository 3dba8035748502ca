"""Offline rank-r extraction of the 16-bit branch, float64 (test infrastructure: only the
tests, the smoke check and the bench's CPU baseline use this package).

SVDQuant explainer §3: the weight is split into a low-rank part, kept in 16 bits, made of
its leading singular directions, and a residual that is quantized to 4 bits.  With the
weight given as Wt [N][K] (row n = output n):

    Wt = U diag(s) V^T (LAPACK SVD, s descending),
    L2 = U_r diag(s_r)^1/2            [N][r]
    L1 = diag(s_r)^1/2 V_r^T          [r][K]
    R  = Wt - L2_16 L1_16             with L1_16, L2_16 the fp16 factors the branch uses,

so X R^T + (X L1_16^T) L2_16^T = X Wt^T exactly before R is quantized.  The even split of
s between the two factors is this package's reading (the pages only say the branch is
low rank and 16-bit); the product L2 L1 does not depend on it.
"""

import numpy as np


def svd_lowrank_f64(Wt, r):
    """(L1 [r][K], L2 [N][r], s [min(N, K)]) in float64, without rounding."""
    Wt = np.asarray(Wt, dtype=np.float64)
    U, s, Vt = np.linalg.svd(Wt, full_matrices=False)
    h = np.sqrt(s[:r])
    return h[:, None] * Vt[:r], U[:, :r] * h[None, :], s


def svd_lowrank(Wt16, r):
    """dict(L1=fp16 [r][K], L2=fp16 [N][r], R=fp16 [N][K] = fp16(Wt - L2 L1) with the
    fp16 factors, R64 = the same in float64 before rounding, s=singular values)."""
    L1, L2, s = svd_lowrank_f64(Wt16, r)
    L1h, L2h = L1.astype(np.float16), L2.astype(np.float16)
    R64 = np.asarray(Wt16, dtype=np.float64) - L2h.astype(np.float64) @ L1h.astype(np.float64)
    return dict(L1=L1h, L2=L2h, R=R64.astype(np.float16), R64=R64, s=s)
