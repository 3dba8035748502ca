"""Seeded synthetic inputs for the activation path and the 4-bit linears.

This module draws random numbers only: activations, transform parameters and
weights.  It holds none of the method's arithmetic (no transform, no quantizer, no
fold) and is the one module that both the oracle-side tests and the GPU-side
tests/bench use.

Recipe (stands in for the activations and weights of the pages' models, PixArt-Sigma,
SANA, FLUX.1 and CogVideoX, which are not available):

* activations X[M, K] = fp16( Z * s + mu_tok (+ drift_frame) ), Z ~ N(0, 1),
  s = 50 on 12 random outlier channels and 1 elsewhere, mu_tok ~ N(0, sigma_mu^2)
  per token (adaLN-like shift), and for the video workload a per-frame drift
  N(0, 1) over frame-major tokens;
* Kronecker factors A = Q_A diag(u_A), B = Q_B diag(u_B) with Q Haar-random
  orthogonal (QR of a Gaussian matrix with the sign of R's diagonal folded in) and
  u ~ U[0.5, 2]; one pair per layer (or, for per-block factors, one independent pair per
  block index); float32;
* RPBH parameters: a uniform random permutation of K and uniform random +-1 signs;
* power-of-two channel exponents: round(log2(outlier scale)) = 6 on the planted
  outlier channels of the activations and 0 elsewhere (the channels the scaling is
  meant for), or, to exercise every exponent, uniform integers in 0..15;
* weights W ~ N(0, 1/K), low-rank factors L1 ~ N(0, 1/K), L2 ~ N(0, 1/K), fp16,
  in the [out][in] layout: W as [N][K], L1 as [r][K], L2 as [N][r];
* for the low-rank extraction: W = N(0, 1/K) plus r planted directions whose strengths
  fall geometrically from 16 to 4 times the bulk's spectral edge, and a Gaussian
  starting block for the subspace iteration;

Every stream comes from numpy's PCG64 seeded by a SeedSequence of
(config seed, stream tag, sizes), so any piece can be drawn on its own.
"""

import numpy as np

# The five workloads: shapes, transform, formats, rank and activation statistics.
CONFIGS = {
    0: dict(name="pixart-sigma single linear", M=256,
            layers=[("linear", 1152, 1152)],
            xform="kron", fmt="mxfp4", wfmt="mxfp4", rank=32, center=False,
            sigma_mu=2.0, frames=None),
    1: dict(name="pixart-sigma DiT block linears, 1024px, batch 2", M=2 * 4096,
            layers=[("qkv", 1152, 3456), ("proj", 1152, 1152), ("fc1", 1152, 4608), ("fc2", 4608, 1152)],
            xform="kron", fmt="mxfp4", wfmt="mxfp4", rank=32, center=False,
            sigma_mu=2.0, frames=None),
    2: dict(name="sana-like linears, 1024 tokens, batch 4", M=4 * 1024,
            layers=[("qkv", 2240, 6720), ("fc1", 2240, 5600), ("fc2", 5600, 2240)],
            xform="rpbh", fmt="lm4", wfmt="lm2", rank=0, center=False,
            sigma_mu=2.0, frames=None),
    3: dict(name="flux.1-like joint block, centred", M=4096 + 512,
            layers=[("qkv", 3072, 9216), ("fc1", 3072, 12288), ("fc2", 12288, 3072)],
            xform="rpbh", fmt="mxfp4", wfmt="mxfp4", rank=32, center=True,
            sigma_mu=4.0, frames=None),
    4: dict(name="cogvideox-like video DiT linears", M=13 * 1350,
            layers=[("attn", 3072, 3072), ("fc1", 3072, 12288)],
            xform="kron", fmt="mxfp4", wfmt="mxfp4", rank=32, center=False,
            sigma_mu=2.0, frames=13),
}

N_OUTLIERS = 12
OUTLIER_SCALE = 50.0

(_TAG_ACT, _TAG_KRON, _TAG_RPBH, _TAG_W, _TAG_DENSE, _TAG_PTS, _TAG_KRON_BLOCKS, _TAG_LOWRANK_W,
 _TAG_OMEGA) = 1, 2, 3, 4, 5, 6, 7, 8, 9


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _activation_draws(M, K, seed, sigma_mu, n_outliers):
    rng = _rng(seed, _TAG_ACT, M, K)
    mu_tok = rng.normal(0.0, sigma_mu, size=M)
    z = rng.standard_normal((M, K), dtype=np.float64)
    cols = rng.choice(K, size=min(n_outliers, K), replace=False)
    return rng, mu_tok, z, cols


def activations(M, K, seed, sigma_mu=2.0, frames=None, n_outliers=N_OUTLIERS, outlier_scale=OUTLIER_SCALE):
    """fp16 [M, K] activations (see module docstring)."""
    rng, mu_tok, z, cols = _activation_draws(M, K, seed, sigma_mu, n_outliers)
    z[:, cols] *= outlier_scale
    z += mu_tok[:, None]
    if frames:
        drift = rng.standard_normal(frames)
        per = -(-M // frames)
        z += np.repeat(drift, per)[:M, None]
    return z.astype(np.float16)


def outlier_channels(M, K, seed, sigma_mu=2.0, n_outliers=N_OUTLIERS):
    """The channels that activations(M, K, seed, ...) scaled up (sorted int array)."""
    return np.sort(_activation_draws(M, K, seed, sigma_mu, n_outliers)[3])


def pts_exponents(K, channels=None, shift=None, seed=None):
    """int8 [K] power-of-two exponents.  With `channels`: `shift` (default
    round(log2(OUTLIER_SCALE))) on those channels, 0 elsewhere.  With `seed` instead:
    uniform integers in 0..15 on every channel."""
    if seed is not None:
        return _rng(seed, _TAG_PTS, K).integers(0, 16, size=K).astype(np.int8)
    e = np.zeros(K, dtype=np.int8)
    if channels is not None:
        e[np.asarray(channels)] = int(round(np.log2(OUTLIER_SCALE))) if shift is None else int(shift)
    return e


def _haar(rng, n):
    g = rng.standard_normal((n, n))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def kron_factors(seed, layer):
    """(A [4, 4], B [8, 8]) float32 for one layer."""
    rng = _rng(seed, _TAG_KRON, layer)
    A = _haar(rng, 4) * rng.uniform(0.5, 2.0, size=4)[None, :]
    B = _haar(rng, 8) * rng.uniform(0.5, 2.0, size=8)[None, :]
    return A.astype(np.float32), B.astype(np.float32)


def kron_block_factors(seed, layer, nb):
    """Per-block factors (A [nb, 4, 4], B [nb, 8, 8]) float32: the Kronecker recipe drawn
    independently for each block index."""
    rng = _rng(seed, _TAG_KRON_BLOCKS, layer, nb)
    A = np.stack([_haar(rng, 4) * rng.uniform(0.5, 2.0, size=4)[None, :] for _ in range(nb)])
    B = np.stack([_haar(rng, 8) * rng.uniform(0.5, 2.0, size=8)[None, :] for _ in range(nb)])
    return A.astype(np.float32), B.astype(np.float32)


def dense_block(seed, layer):
    """Dense 32x32 block transform P (float32), the same recipe as the Kronecker factors at
    full size: Haar-orthogonal times column scales drawn from U[0.5, 2]."""
    rng = _rng(seed, _TAG_DENSE, layer)
    return (_haar(rng, 32) * rng.uniform(0.5, 2.0, size=32)[None, :]).astype(np.float32)


def rpbh_params(K, seed, layer):
    """(perm int32 [K], sign int8 [K] of +-1) for one layer."""
    rng = _rng(seed, _TAG_RPBH, layer, K)
    perm = rng.permutation(K).astype(np.int32)
    sign = rng.choice(np.array([-1, 1], dtype=np.int8), size=K)
    return perm, sign


def weights(K, N, seed, layer, rank=32):
    """(W [N, K], L1 [rank, K] or None, L2 [N, rank] or None), fp16, [out][in] layout."""
    rng = _rng(seed, _TAG_W, layer, K, N)
    sd = 1.0 / np.sqrt(K)
    W = rng.normal(0.0, sd, size=(N, K)).astype(np.float16)
    if rank == 0:
        return W, None, None
    L1 = rng.normal(0.0, sd, size=(rank, K)).astype(np.float16)
    L2 = rng.normal(0.0, sd, size=(N, rank)).astype(np.float16)
    return W, L1, L2


def planted_lowrank_weights(K, N, seed, layer, r, top=16.0, bottom=4.0):
    """fp16 Wt [N][K] = G + U diag(s) V^T: G ~ N(0, 1/K) and r planted directions (U, V
    with orthonormal columns from QR of Gaussians) whose strengths fall geometrically from
    `top` to `bottom` times the bulk's spectral edge 1 + sqrt(N / K) -- weights whose
    leading singular directions stand out, as the low-rank branch assumes."""
    rng = _rng(seed, _TAG_LOWRANK_W, layer, K, N, r)
    G = rng.normal(0.0, 1.0 / np.sqrt(K), size=(N, K))
    U, _ = np.linalg.qr(rng.standard_normal((N, r)))
    V, _ = np.linalg.qr(rng.standard_normal((K, r)))
    edge = 1.0 + np.sqrt(N / K)
    s = edge * np.geomspace(top, bottom, r)
    return (G + (U * s[None, :]) @ V.T).astype(np.float16)


def gaussian_block(K, l, seed):
    """float32 [K][l] of N(0, 1): the starting block of randomized subspace iteration."""
    return _rng(seed, _TAG_OMEGA, K, l).standard_normal((K, l)).astype(np.float32)


def xform_for(cfg_idx, layer, K):
    """Transform descriptor dict for layer `layer` of config `cfg_idx`."""
    cfg = CONFIGS[cfg_idx]
    if cfg["xform"] == "kron":
        A, B = kron_factors(cfg_idx, layer)
        return {"kind": "kron", "A": A, "B": B}
    perm, sign = rpbh_params(K, cfg_idx, layer)
    return {"kind": "rpbh", "perm": perm, "sign": sign}


def layer_inputs(cfg_idx, layer, M=None):
    """Everything one layer of a config needs: X, transform, W, L1, L2 (numpy)."""
    cfg = CONFIGS[cfg_idx]
    name, K, N = cfg["layers"][layer]
    M = cfg["M"] if M is None else M
    X = activations(M, K, cfg_idx, cfg["sigma_mu"], cfg["frames"])
    W, L1, L2 = weights(K, N, cfg_idx, layer, cfg["rank"])
    return dict(name=name, M=M, K=K, N=N, X=X, xform=xform_for(cfg_idx, layer, K), W=W, L1=L1, L2=L2,
                fmt=cfg["fmt"], wfmt=cfg["wfmt"], center=cfg["center"], rank=cfg["rank"])
