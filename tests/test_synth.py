"""The seeded input generator: determinism and the distribution it promises."""

import numpy as np

import synth


def test_deterministic_and_independent_streams():
    a = synth.activations(64, 256, seed=3, sigma_mu=2.0)
    b = synth.activations(64, 256, seed=3, sigma_mu=2.0)
    c = synth.activations(64, 256, seed=4, sigma_mu=2.0)
    assert a.dtype == np.float16 and np.array_equal(a, b) and not np.array_equal(a, c)
    A1, B1 = synth.kron_factors(0, 0)
    A2, B2 = synth.kron_factors(0, 1)
    assert A1.dtype == np.float32 and not np.array_equal(A1, A2)


def test_activation_moments():
    M, K = 2048, 512
    X = synth.activations(M, K, seed=0, sigma_mu=2.0).astype(np.float64)
    col_sd = X.std(axis=0)
    outliers = np.argsort(col_sd)[-12:]
    assert np.all(col_sd[outliers] > 40) and np.median(col_sd) < 3.0
    normal = np.setdiff1d(np.arange(K), outliers)
    mu = X[:, normal].mean(axis=1)
    assert abs(mu.std() - 2.0) < 0.15               # per-token shift N(0, 2^2)
    resid = X[:, normal] - mu[:, None]
    assert abs(resid.std() - 1.0) < 0.02


def test_video_frame_drift():
    M, K = 13 * 40, 64
    X = synth.activations(M, K, seed=4, sigma_mu=0.0, frames=13, n_outliers=0).astype(np.float64)
    fm = X.reshape(13, 40, K).mean(axis=(1, 2))
    assert np.std(fm) > 0.3                         # N(0, 1) drift per frame
    assert np.all(np.abs(X.reshape(13, 40, K).mean(axis=2) - fm[:, None]) < 0.7)


def test_factors_haar_times_diag():
    A, B = synth.kron_factors(0, 0)
    for F, n in ((A, 4), (B, 8)):
        col = np.linalg.norm(F.astype(np.float64), axis=0)       # = the diagonal factor
        assert np.all((col >= 0.5 - 1e-6) & (col <= 2.0 + 1e-6))
        Q = F / col[None, :]
        assert np.allclose(Q.T @ Q, np.eye(n), atol=1e-6)


def test_rpbh_params_and_weights():
    perm, sign = synth.rpbh_params(3072, 3, 0)
    assert np.array_equal(np.sort(perm), np.arange(3072)) and set(np.unique(sign)) == {-1, 1}
    W, L1, L2 = synth.weights(1152, 64, 0, 0, rank=32)
    assert W.shape == (64, 1152) and L1.shape == (32, 1152) and L2.shape == (64, 32)
    assert abs(W.astype(np.float64).std() * np.sqrt(1152) - 1.0) < 0.02
    W2, n1, n2 = synth.weights(2240, 8, 2, 0, rank=0)
    assert n1 is None and n2 is None


def test_config_table_matches_workloads():
    c = synth.CONFIGS
    assert c[0]["M"] == 256 and c[1]["M"] == 8192 and c[2]["M"] == 4096
    assert c[3]["M"] == 4608 and c[4]["M"] == 17550
    assert [l[1:] for l in c[3]["layers"]] == [(3072, 9216), (3072, 12288), (12288, 3072)]
    assert c[3]["center"] and c[3]["xform"] == "rpbh" and c[2]["fmt"] == "lm4"


def test_outlier_channels_are_the_scaled_ones():
    """outlier_channels replays the activations' draw: exactly the channels with the large
    spread, and the power-of-two exponents land on them."""
    M, K = 512, 384
    X = synth.activations(M, K, seed=5, sigma_mu=2.0).astype(np.float64)
    ch = synth.outlier_channels(M, K, seed=5, sigma_mu=2.0)
    assert np.array_equal(np.sort(np.argsort(X.std(axis=0))[-12:]), ch)
    e = synth.pts_exponents(K, ch)
    assert e.dtype == np.int8 and np.all(e[ch] == 6) and np.count_nonzero(e) == 12
    r = synth.pts_exponents(K, seed=9)
    assert r.min() >= 0 and r.max() <= 15 and np.array_equal(r, synth.pts_exponents(K, seed=9))


def test_block_factors_and_planted_weights():
    A, B = synth.kron_block_factors(1, 0, 6)
    assert A.shape == (6, 4, 4) and B.shape == (6, 8, 8) and not np.array_equal(A[0], A[1])
    for a in A.astype(np.float64):                  # Haar times positive column scales
        q = a / np.linalg.norm(a, axis=0)[None, :]
        assert np.allclose(q.T @ q, np.eye(4), atol=1e-5)
    W = synth.planted_lowrank_weights(512, 128, 2, 0, 8).astype(np.float64)
    s = np.linalg.svd(W, compute_uv=False)
    edge = 1.0 + np.sqrt(128 / 512)
    assert s[7] > 3.0 * edge and s[8] < 1.3 * edge   # the planted directions stand out of the bulk
    om = synth.gaussian_block(96, 24, 3)
    assert om.shape == (96, 24) and om.dtype == np.float32 and abs(om.std() - 1.0) < 0.05
