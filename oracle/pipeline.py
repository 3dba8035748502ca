"""The online activation path and the offline weight fold, end to end, float64.

transform_quantize: optional per-token centring (CentriQ page, arXiv abstract) ->
32-element block transform (KroQuant §02 Kronecker, or OrbitQuant §03 RPBH) ->
4-bit quantization (MXFP4 per KroQuant §03, or the per-token Lloyd-Max codebook of
OrbitQuant §03 / CentriQ's closed-form scale) -> packed codes.

fold_weights: W' = P^-1 W offline (KroQuant §01, OrbitQuant §03), quantized along K
with the same rules (MXFP4) or to 2-bit Lloyd-Max groups; plus the rank-1 restore
vector wbar = 1^T W (CentriQ abstract: a rank-1 high-precision term gives back what
the centring removed, since (x - mu 1^T) W + mu (1^T W) = x W).

Transform descriptors are plain dicts:
  {"kind": "kron", "A": float32 [4, 4], "B": float32 [8, 8]}
  {"kind": "rpbh", "perm": int [K], "sign": int8 [K] (+-1)}
  {"kind": "dense", "P": float32 [32, 32]}     (y_b = x_b . P)
  {"kind": "kron_blocks", "A": float32 [K/32, 4, 4], "B": float32 [K/32, 8, 8]}
                                               (y_b = x_b . kron(A_b, B_b))
  {"kind": "none"}
Any of them except "rpbh" may carry "pts": int [K] of power-of-two exponents (DMQ
explainer, channel-wise power-of-two scaling): the activation path first replaces
x_k by fp16(x_k 2^-e_k), and the fold scales weight input channel k by 2^e_k.
"""

import numpy as np

from . import lloyd_max, mxfp4, transforms


def token_mean_f16(x):
    """Per-token mean over all K channels in float64, rounded to fp16 (RNE).

    The stored fp16 mean is what centring subtracts, so the rank-1 restore is exact
    by construction (CentriQ abstract).
    """
    x = np.asarray(x, dtype=np.float64)
    return np.mean(x, axis=1).astype(np.float16)


def centre(x, mu_f16):
    """x - mu (float64, exact for fp16 inputs)."""
    return np.asarray(x, dtype=np.float64) - np.asarray(mu_f16, dtype=np.float64)[:, None]


def apply_pts(x, pts):
    """Channel-wise power-of-two scaling of the activations (DMQ explainer, PTS): channel
    k is divided by 2^pts[k].  The pages call it a bit shift of 16-bit values, so the
    result stays fp16: the scaling is exact unless it lands below the fp16 normal range,
    where numpy's float64 -> float16 conversion rounds to nearest even."""
    e = np.asarray(pts, dtype=np.int64)
    return np.ldexp(np.asarray(x, dtype=np.float64), -e[None, :]).astype(np.float16).astype(np.float64)


def apply_transform(x, xform):
    kind = xform["kind"]
    if kind == "kron":
        return transforms.apply_block_matrix(x, transforms.kron_block_matrix(xform["A"], xform["B"]))
    if kind == "rpbh":
        return transforms.rpbh_apply(x, xform["perm"], xform["sign"])
    if kind == "dense":
        return transforms.apply_block_matrix(x, np.asarray(xform["P"], dtype=np.float64))
    if kind == "kron_blocks":
        return transforms.apply_block_matrices(x, transforms.kron_block_matrices(xform["A"], xform["B"]))
    if kind == "none":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(kind)


def transform_quantize(X_f16, xform, fmt="mxfp4", center=False, mu_f16=None):
    """Quantize activations X (fp16 [M, K]).

    fmt "mxfp4": returns dict(codes=u8 [M, K/2] packed, scales=u8 [M, K/32], mu=f16 [M] or None,
                              y=float64 transformed values, codes_unpacked, exponents)
    fmt "lm4":   returns dict(codes=u8 [M, K/2] packed, scales=f32 [M], mu=..., y=..., codes_unpacked)
    If mu_f16 is given it is used instead of the oracle's own mean (tie re-evaluation).
    """
    x = np.asarray(X_f16, dtype=np.float64)
    mu = None
    if xform.get("pts") is not None:
        if center or xform["kind"] == "rpbh":
            raise ValueError("power-of-two channel scaling is defined here without centring or RPBH")
        x = apply_pts(x, xform["pts"])
    if center:
        mu = token_mean_f16(x) if mu_f16 is None else np.asarray(mu_f16, dtype=np.float16)
        x = centre(x, mu)
    y = apply_transform(x, xform)
    if fmt == "mxfp4":
        codes, scale_bytes, e = mxfp4.quantize_blocks(y)
        return dict(codes=mxfp4.pack_nibbles(codes), scales=scale_bytes, mu=mu, y=y,
                    codes_unpacked=codes, exponents=e)
    if fmt == "lm4":
        codes, s = lloyd_max.lm4_token_quantize(y)
        return dict(codes=mxfp4.pack_nibbles(codes), scales=s, mu=mu, y=y, codes_unpacked=codes)
    raise ValueError(fmt)


def inverse_fold(W_out_in, xform):
    """W'^T = (P^-1 D W)^T as [N][K] float64, for W given as [N][K] (row n = column n of W);
    D = diag(2^pts) when the descriptor carries power-of-two exponents, else the identity."""
    kind = xform["kind"]
    if xform.get("pts") is not None:
        if kind == "rpbh":
            raise ValueError("power-of-two channel scaling is defined here without RPBH")
        e = np.asarray(xform["pts"], dtype=np.int64)
        W_out_in = np.ldexp(np.asarray(W_out_in, dtype=np.float64), e[None, :])
    if kind == "kron":
        return transforms.fold_kron(W_out_in, xform["A"], xform["B"])
    if kind == "rpbh":
        return transforms.fold_rpbh(W_out_in, xform["perm"], xform["sign"])
    if kind == "dense":
        return transforms.fold_dense(W_out_in, xform["P"])
    if kind == "kron_blocks":
        return transforms.fold_kron_blocks(W_out_in, xform["A"], xform["B"])
    if kind == "none":
        return np.asarray(W_out_in, dtype=np.float64)
    raise ValueError(kind)


def column_sums_f16(W_out_in):
    """wbar_n = sum_k W[k, n] in float64, rounded to fp16."""
    return np.asarray(W_out_in, dtype=np.float64).sum(axis=1).astype(np.float16)


def fold_weights(W_out_in_f16, xform, fmt="mxfp4"):
    """Offline fold: returns dict(wcodes, wscales, wbar, wt=W'^T float64, codes_unpacked)."""
    wt = inverse_fold(W_out_in_f16, xform)
    wbar = column_sums_f16(W_out_in_f16)
    if fmt == "mxfp4":
        codes, scale_bytes, e = mxfp4.quantize_blocks(wt)
        return dict(wcodes=mxfp4.pack_nibbles(codes), wscales=scale_bytes, wbar=wbar, wt=wt,
                    codes_unpacked=codes, exponents=e)
    if fmt == "lm2":
        codes, s = lloyd_max.w2_group_quantize(wt)
        return dict(wcodes=lloyd_max.pack_2bit(codes), wscales=s, wbar=wbar, wt=wt,
                    codes_unpacked=codes)
    raise ValueError(fmt)
