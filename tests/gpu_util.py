"""Shared helpers of the GPU parity tests: error bounds of the kernels' float32
arithmetic (used to classify ties), and running the oracle on the same inputs."""

import numpy as np

from oracle import mxfp4, pipeline, ties, transforms

U = 2.0 ** -24

# Forward-error bounds of the kernels' float32 arithmetic per output element, by path:
#  Kronecker (shared or per-block factors) or dense P, no centring (matrix cores): P
#      (A (x) B formed in float32, or given) split into fp16 hi + lo parts (~2^-21
#      relative), 64 exact products accumulated in float32;
#  Kronecker or identity with centring, and Lloyd-Max (vector units): an 8-term FMA chain
#      feeding a 4-term chain, plus the centring subtraction;
#  RPBH, MXFP4 (matrix cores): 32 exact +-1 products of the UNCENTRED inputs accumulated in
#      float32, the centring applied to output 0 of each block afterwards (subtracting
#      32 mu), then the rounded 1/sqrt(32) and the final product;
#  RPBH, Lloyd-Max (vector units): five butterfly stages, 1/sqrt(32), the product, and
#      the centring subtraction;
#  identity without centring (matrix cores, with or without the power-of-two shift): each
#      output is one fp16 input times 1.0 plus exact zeros, so the float32 value is exact
#      and no tie is allowed (n = 0).
def _path(kind, center, fmt):
    if kind in ("dense", "kron_blocks"):
        return ("uncentred", 80)
    if kind == "kron":
        return ("uncentred", 80) if (not center and fmt == "mxfp4") else ("centred", 14)
    if kind == "rpbh":
        return ("uncentred", 36) if fmt == "mxfp4" else ("centred", 9)
    return ("uncentred", 0) if (not center and fmt == "mxfp4") else ("centred", 2)


def abs_transform(x_abs, xform):
    """sum_i |x_i| |P_ik| (the quantity the float32 error bound scales with)."""
    kind = xform["kind"]
    if kind == "kron":
        P = np.abs(transforms.kron_block_matrix(xform["A"], xform["B"]))
        return transforms.apply_block_matrix(x_abs, P)
    if kind == "rpbh":
        u = x_abs[:, np.asarray(xform["perm"], dtype=np.int64)]
        return transforms.apply_block_matrix(u, np.abs(transforms.hadamard32())) / np.sqrt(32.0)
    if kind == "dense":
        return transforms.apply_block_matrix(x_abs, np.abs(np.asarray(xform["P"], dtype=np.float64)))
    if kind == "kron_blocks":
        return transforms.apply_block_matrices(x_abs, np.abs(transforms.kron_block_matrices(xform["A"], xform["B"])))
    return x_abs


def tau_for(x_c, xform, center, fmt="mxfp4", x_raw=None, mu=None):
    """Per-element error bound of the kernel that handles (transform, centring, format).
    x_c: the centred input (or the raw input when not centring); x_raw, mu: the raw input
    and the fp16 means, needed for the paths that centre after the transform."""
    which, n = _path(xform["kind"], center, fmt)
    if which == "centred" or not center:
        return ties.gamma_tau(n, abs_transform(np.abs(x_c), xform))
    base = abs_transform(np.abs(np.asarray(x_raw, dtype=np.float64)), xform)
    corr = np.zeros_like(base)
    corr[:, 0::32] = 32.0 * np.abs(np.asarray(mu, dtype=np.float64))[:, None] / np.sqrt(32.0)
    return ties.gamma_tau(n, base + corr)


def oracle_activation_reference(X16, xform, center, mu_gpu=None, fmt="mxfp4"):
    """Exact transformed values y (float64) and the kernel's error bound tau, using the
    kernel's mean where it differs from the oracle's only by a rounding tie."""
    X = X16.astype(np.float64)
    mu = None
    if center:
        mu = pipeline.token_mean_f16(X16)
        if mu_gpu is not None:
            mu = mu_gpu.copy()
        xc = pipeline.centre(X, mu)
    else:
        xc = X
    if xform.get("pts") is not None:
        xc = pipeline.apply_pts(xc, xform["pts"])      # fp16 values: the kernel's own inputs
    y = pipeline.apply_transform(xc, xform)
    return y, tau_for(xc, xform, center, fmt, x_raw=X, mu=mu), mu


def check_mu(X16, mu_gpu):
    """fp16 means: equal to the oracle's, or an adjacent rounding at a tie.  Returns the
    number of ties; raises on any other difference."""
    ref = pipeline.token_mean_f16(X16)
    diff = np.flatnonzero(ref.view(np.uint16) != mu_gpu.view(np.uint16))
    K = X16.shape[1]
    for m in diff:
        n_terms = K + 16
        assert ties.mean_tie(X16[m], mu_gpu[m], ref[m], n_terms), (m, float(mu_gpu[m]), float(ref[m]))
    return len(diff)


def assert_mx_parity(codes_gpu_packed, scales_gpu, y, tau, max_frac=1e-4, label=""):
    codes = mxfp4.unpack_nibbles(codes_gpu_packed)
    rep = ties.classify_mxfp4(codes, scales_gpu, y, tau)
    frac = rep["code_mismatch"] / rep["codes"]
    msg = (f"{label}: code mismatches {rep['code_mismatch']}/{rep['codes']} (ties {rep['code_ties']}), "
           f"scale mismatches {rep['scale_mismatch']} (ties {rep['scale_ties']}), errors {rep['errors'][:5]}")
    print(msg)
    for t in rep["ties"][:10]:
        print("  tie", t)
    assert not rep["errors"], msg
    assert frac <= max_frac, msg
    assert rep["scale_mismatch"] / rep["blocks"] <= max_frac, msg
    return rep
