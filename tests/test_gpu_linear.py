"""GPU parity of the offline fold and of the 4-bit linear (W4A4 + low-rank + rank-1, and
W2A4) against the oracle.

The fold's codes follow the same tie rule as the activations.  The linear is checked on
the kernel's own packed operands (so code ties cannot leak into it): the oracle
dequantizes them in float64 and adds the branches exactly; the fp16 result must be within
2e-3 relative Frobenius error.
"""

import numpy as np
import pytest

import synth
from oracle import linear, lloyd_max, mxfp4, pipeline, ties, transforms
from tests import gpu_util
from tests.test_gpu_transform import _dev_xform

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _fold(kq, W16, xf, fmt):
    import torch
    W = torch.from_numpy(W16).cuda()
    dxf = _dev_xform(kq, torch, xf, W16.shape[1])
    wc, ws, wbar = kq.fold_inverse_into_weights_nk(W, dxf, fmt=fmt)
    torch.cuda.synchronize()
    return wc, ws, wbar


def _wbar_check(W16, wbar_gpu):
    """The fold's column sums against the oracle's: the device sums in float64 and rounds
    once, so they must be the same fp16 values (a float64 summation-order difference could
    only matter for a sum within 2^-40 of an fp16 rounding midpoint; none is allowed)."""
    ref = pipeline.column_sums_f16(W16)
    assert np.array_equal(ref.view(np.uint16), wbar_gpu.view(np.uint16))


@pytest.mark.parametrize("cfg,layer,nrows", [(0, 0, 1152), (1, 1, 200), (3, 2, 96), (4, 0, 160), (1, 3, 80)])
def test_fold_mxfp4_matches_oracle(kq, cfg, layer, nrows):
    c = synth.CONFIGS[cfg]
    _, K, N = c["layers"][layer]
    W16, _, _ = synth.weights(K, N, cfg, layer, 0)
    W16 = np.ascontiguousarray(W16[:nrows])
    xf = synth.xform_for(cfg, layer, K)
    wc, ws, wbar = _fold(kq, W16, xf, "mxfp4")
    wt = pipeline.inverse_fold(W16, xf)
    if xf["kind"] == "kron":
        # w'_b = P^-1 w_b, so the bound scales with sum_k |P^-1[j][k]| |w_k| = (|w| |P^-T|)_j
        inv_t = {"kind": "kron", "A": np.linalg.inv(xf["A"].astype(np.float64)).T,
                 "B": np.linalg.inv(xf["B"].astype(np.float64)).T}
        tau = ties.gamma_tau(13, gpu_util.abs_transform(np.abs(W16.astype(np.float64)), inv_t))
    else:   # W'^T = W^T R, five butterfly stages, 1/sqrt(32) and the product
        tau = ties.gamma_tau(8, gpu_util.abs_transform(np.abs(W16.astype(np.float64)), xf))
    gpu_util.assert_mx_parity(wc.cpu().numpy(), ws.cpu().numpy(), wt, tau, label=f"fold cfg{cfg} layer{layer}")
    _wbar_check(W16, wbar.cpu().numpy())


def test_fold_dense_matches_oracle(kq):
    """The fold with a dense P: P^-1 by Gauss-Jordan on the device (float64), then a float32
    product per 32-block; the bound scales with (|w| |P^-T|)."""
    K, N = 1152, 160
    W16, _, _ = synth.weights(K, N, 13, 0, 0)
    P = synth.dense_block(13, 0)
    xf = {"kind": "dense", "P": P}
    wc, ws, wbar = _fold(kq, W16, xf, "mxfp4")
    wt = pipeline.inverse_fold(W16, xf)
    inv_t = {"kind": "dense", "P": np.linalg.inv(P.astype(np.float64)).T}
    tau = ties.gamma_tau(36, gpu_util.abs_transform(np.abs(W16.astype(np.float64)), inv_t))
    gpu_util.assert_mx_parity(wc.cpu().numpy(), ws.cpu().numpy(), wt, tau, label="fold dense")
    _wbar_check(W16, wbar.cpu().numpy())


def test_w4a4_dense_block_linear(kq):
    """The whole path with a dense P: transform + quantize, fold, low-rank branch, W4A4
    linear; the oracle dequantizes the kernel's own packed operands."""
    import torch
    M, K, N, r = 300, 1152, 512, 32
    X16 = synth.activations(M, K, 14, 2.0)
    W16, L1, L2 = synth.weights(K, N, 14, 0, r)
    xf = {"kind": "dense", "P": synth.dense_block(14, 0)}
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, _ = kq.transform_quantize(X, dxf, fmt="mxfp4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="mxfp4")
    T = kq.lowrank_down(X, torch.from_numpy(L1).cuda())
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=torch.from_numpy(np.ascontiguousarray(L2)).cuda())
    torch.cuda.synchronize()
    ref = linear.w4a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), X16, L1, L2,
                             None, None)
    err = linear.rel_frobenius(Y.cpu().numpy(), ref)
    print(f"dense-P linear rel frobenius {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("kind", ["kron", "dense", "none"])
def test_fold_pts_matches_oracle(kq, kind):
    """The fold with power-of-two channel exponents: W scaled by 2^e along its input channel
    (exact), then P^-1; wbar stays the sum of the unscaled weights."""
    K, N = 1152, 160
    W16, _, _ = synth.weights(K, N, 15, 0, 0)
    xf = {"kind": kind, "pts": synth.pts_exponents(K, seed=15)}
    if kind == "kron":
        xf["A"], xf["B"] = synth.kron_factors(15, 0)
        inv_t = {"kind": "kron", "A": np.linalg.inv(xf["A"].astype(np.float64)).T,
                 "B": np.linalg.inv(xf["B"].astype(np.float64)).T}
        n = 13
    elif kind == "dense":
        xf["P"] = synth.dense_block(15, 0)
        inv_t = {"kind": "dense", "P": np.linalg.inv(xf["P"].astype(np.float64)).T}
        n = 36
    else:
        inv_t, n = {"kind": "none"}, 2
    wc, ws, wbar = _fold(kq, W16, xf, "mxfp4")
    wt = pipeline.inverse_fold(W16, xf)
    wd = np.ldexp(np.abs(W16.astype(np.float64)), xf["pts"].astype(np.int64)[None, :])
    tau = ties.gamma_tau(n, gpu_util.abs_transform(wd, inv_t))
    gpu_util.assert_mx_parity(wc.cpu().numpy(), ws.cpu().numpy(), wt, tau, label=f"fold pts {kind}")
    _wbar_check(W16, wbar.cpu().numpy())


@pytest.mark.parametrize("kind", ["kron", "dense"])
def test_w4a4_pts_linear(kq, kind):
    """The whole path with power-of-two scaling on the outlier channels: the linear of the
    kernel's packed operands against the oracle, and the quantized product against the
    exact X W.  The scaling cancels between the two sides, so the 4-bit error stays of
    order one (the oracle's own figure on these inputs is 0.64 for Kronecker and 0.39 for
    dense P: the weights of the scaled channels grow by 2^6); a shift applied the wrong
    way on either side would give errors of order 2^12."""
    import torch
    M, K, N, r = 260, 3072, 384, 32
    X16 = synth.activations(M, K, 16, 2.0)
    W16, L1, L2 = synth.weights(K, N, 16, 0, r)
    xf = {"kind": kind, "pts": synth.pts_exponents(K, synth.outlier_channels(M, K, 16, 2.0))}
    if kind == "kron":
        xf["A"], xf["B"] = synth.kron_factors(16, 0)
    else:
        xf["P"] = synth.dense_block(16, 0)
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, _ = kq.transform_quantize(X, dxf, fmt="mxfp4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="mxfp4")
    T = kq.lowrank_down(X, torch.from_numpy(L1).cuda())
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=torch.from_numpy(np.ascontiguousarray(L2)).cuda())
    torch.cuda.synchronize()
    ref = linear.w4a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), X16, L1, L2,
                             None, None)
    err = linear.rel_frobenius(Y.cpu().numpy(), ref)
    exact = X16.astype(np.float64) @ W16.astype(np.float64).T + linear.lowrank_term(X16, L1, L2)
    qerr = linear.rel_frobenius(Y.cpu().numpy(), exact)
    print(f"pts {kind} linear rel frobenius {err:.3e}; against exact X W {qerr:.3e}")
    assert err <= TOL
    assert qerr < 1.0


@pytest.mark.parametrize("K,N,pts", [(1152, 160, False), (96, 40, False), (3072, 64, True)])
def test_fold_kron_blocks_matches_oracle(kq, K, N, pts):
    """The fold with per-block factors: each block's A_b (x) B_b formed in float64 and
    inverted on the device by Gauss-Jordan, then a float32 product per block."""
    W16, _, _ = synth.weights(K, N, 19, 0, 0)
    A, B = synth.kron_block_factors(19, 0, K // 32)
    xf = {"kind": "kron_blocks", "A": A, "B": B}
    wd = np.abs(W16.astype(np.float64))
    if pts:
        xf["pts"] = synth.pts_exponents(K, seed=19)
        wd = np.ldexp(wd, xf["pts"].astype(np.int64)[None, :])
    wc, ws, wbar = _fold(kq, W16, xf, "mxfp4")
    wt = pipeline.inverse_fold(W16, xf)
    Pinv = np.linalg.inv(transforms.kron_block_matrices(A, B))
    tau = ties.gamma_tau(36, transforms.apply_block_matrices(wd, np.abs(np.transpose(Pinv, (0, 2, 1)))))
    gpu_util.assert_mx_parity(wc.cpu().numpy(), ws.cpu().numpy(), wt, tau, label=f"fold kron_blocks K={K}")
    _wbar_check(W16, wbar.cpu().numpy())


def test_w4a4_kron_blocks_linear(kq):
    """The whole path with per-block factors: transform + quantize, fold, low-rank branch,
    W4A4 linear, against the oracle on the kernel's own packed operands."""
    import torch
    M, K, N, r = 300, 1152, 512, 32
    X16 = synth.activations(M, K, 20, 2.0)
    W16, L1, L2 = synth.weights(K, N, 20, 0, r)
    A, B = synth.kron_block_factors(20, 0, K // 32)
    xf = {"kind": "kron_blocks", "A": A, "B": B}
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, _ = kq.transform_quantize(X, dxf, fmt="mxfp4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="mxfp4")
    T = kq.lowrank_down(X, torch.from_numpy(L1).cuda())
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=torch.from_numpy(np.ascontiguousarray(L2)).cuda())
    torch.cuda.synchronize()
    ref = linear.w4a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), X16, L1, L2,
                             None, None)
    err = linear.rel_frobenius(Y.cpu().numpy(), ref)
    print(f"kron_blocks linear rel frobenius {err:.3e}")
    assert err <= TOL


def test_fold_w2_matches_oracle(kq):
    c = synth.CONFIGS[2]
    _, K, N = c["layers"][0]
    W16, _, _ = synth.weights(K, N, 2, 0, 0)
    W16 = np.ascontiguousarray(W16[:200])
    xf = synth.xform_for(2, 0, K)
    wc, ws, _ = _fold(kq, W16, xf, "lm2")
    codes = lloyd_max.unpack_2bit(wc.cpu().numpy())
    s_gpu = ws.cpu().numpy()
    wt = pipeline.inverse_fold(W16, xf)
    ref_codes, ref_s = lloyd_max.w2_group_quantize(wt)
    tau = ties.gamma_tau(8, gpu_util.abs_transform(np.abs(W16.astype(np.float64)), xf)).reshape(wt.shape)
    # group scales: fp16 of the RMS; differences only at fp16 rounding ties
    g = wt.reshape(wt.shape[0], -1, 32)
    rms = np.sqrt(np.mean(g * g, axis=2))
    ds = np.argwhere(s_gpu.view(np.uint16) != ref_s.view(np.uint16))
    for (n, b) in ds:
        a, bb = float(s_gpu[n, b]), float(ref_s[n, b])
        assert abs(rms[n, b] - 0.5 * (a + bb)) <= 1e-5 * rms[n, b]
    assert len(ds) <= 2
    thr = lloyd_max.thresholds(lloyd_max.LEVELS4)[0]
    s_used = np.repeat(s_gpu.astype(np.float64), 32, axis=1)
    mism = np.argwhere(codes != lloyd_max.sign_magnitude_encode(
        np.where(s_used > 0, wt / np.where(s_used > 0, s_used, 1), 0), np.array([thr])))
    for (n, k) in mism:
        v = abs(wt[n, k]) / s_used[n, k]
        assert abs(v - thr) <= (tau[n, k] / s_used[n, k]) + 4 * gpu_util.U * thr, (n, k, v)
    assert len(mism) / codes.size <= 1e-4


def _linear_case(kq, cfg, layer, M, N=None, rank=None, with_mu=None, K=None, seed_shift=0):
    import torch
    c = synth.CONFIGS[cfg]
    _, K0, N0 = c["layers"][layer]
    K = K0 if K is None else K
    N = N0 if N is None else N
    r = c["rank"] if rank is None else rank
    center = c["center"] if with_mu is None else with_mu
    X16 = synth.activations(M, K, cfg + seed_shift, c["sigma_mu"], c["frames"])
    W16, L1, L2 = synth.weights(K, N, cfg + seed_shift, layer, max(r, 1))
    if r == 0:
        L1 = L2 = None
    else:
        L1, L2 = L1[:r], np.ascontiguousarray(L2[:, :r])
    xf = synth.xform_for(cfg, layer, K) if K == K0 else {"kind": "kron", "A": synth.kron_factors(cfg, layer)[0],
                                                          "B": synth.kron_factors(cfg, layer)[1]}
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, mu = kq.transform_quantize(X, dxf, fmt="mxfp4", center=center)
    wc, ws, wbar = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="mxfp4")
    L1d = None if L1 is None else torch.from_numpy(np.ascontiguousarray(L1)).cuda()
    L2d = None if L2 is None else torch.from_numpy(L2).cuda()
    T = kq.lowrank_down(X, L1d) if r else None
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=L2d, mu=mu, wbar=wbar if center else None)
    torch.cuda.synchronize()
    return dict(X16=X16, W16=W16, L1=L1, L2=L2, xc=xc.cpu().numpy(), xs=xs.cpu().numpy(), wc=wc.cpu().numpy(),
                ws=ws.cpu().numpy(), mu=None if mu is None else mu.cpu().numpy(),
                wbar=None if not center else wbar.cpu().numpy(), Y=Y.cpu().numpy(), xf=xf,
                T=None if T is None else T.cpu().numpy())


def _ref_Y(d, rows=None, cols=None):
    return linear.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"], d["X16"] if d["L1"] is not None else None,
                              d["L1"], d["L2"], d["mu"], d["wbar"], rows=rows, cols=cols)


@pytest.mark.parametrize("cfg,layer,M", [(0, 0, 256), (1, 0, 200), (1, 3, 130), (3, 0, 150), (3, 2, 70), (4, 1, 97)])
def test_w4a4_linear_matches_oracle(kq, cfg, layer, M):
    d = _linear_case(kq, cfg, layer, M)
    ref = _ref_Y(d)
    err = linear.rel_frobenius(d["Y"], ref)
    print(f"cfg{cfg} layer{layer} M={M}: rel frobenius {err:.3e}")
    assert err <= TOL
    # elementwise sanity: no element off by more than a few fp16 ulps of the output scale
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(d["Y"].astype(np.float64) - ref)) <= 0.02 * scale + 1e-3 * np.max(np.abs(ref))


@pytest.mark.parametrize("rank,with_mu", [(0, False), (16, False), (64, True), (32, True)])
def test_w4a4_branch_variants(kq, rank, with_mu):
    d = _linear_case(kq, 1, 1, 77, rank=rank, with_mu=with_mu)
    err = linear.rel_frobenius(d["Y"], _ref_Y(d))
    print(f"rank {rank} mu {with_mu}: {err:.3e}")
    assert err <= TOL


def _check_lowrank(kq, M, K, r, seed=7, workspace="default"):
    """T = fp16(X L1^T): within one fp16 rounding of the exact product (plus the float32
    accumulation bound: K / 8 sequential additions per lane and MFMA block, then the
    split-K partials)."""
    import torch
    X16 = synth.activations(M, K, seed, 2.0)
    _, L1, _ = synth.weights(K, 16, seed, 0, r)
    kw = {} if isinstance(workspace, str) else {"workspace": workspace}
    T = kq.lowrank_down(torch.from_numpy(X16).cuda(), torch.from_numpy(L1).cuda(), **kw)
    torch.cuda.synchronize()
    got = T.cpu().numpy().astype(np.float64)
    exact = X16.astype(np.float64) @ L1.astype(np.float64).T
    bound = np.abs(X16.astype(np.float64)) @ np.abs(L1.astype(np.float64)).T
    err = np.abs(got - exact)
    assert np.all(err <= np.abs(exact) * 2.0 ** -11 + ties.gamma_tau(K // 8 + 16, bound) + 2.0 ** -24)


@pytest.mark.parametrize("M,K,r", [(1, 128, 32), (77, 1152, 16), (301, 3072, 32), (40, 12288, 64), (19, 2240, 32),
                                   (1000, 3072, 64), (4608, 3072, 16), (4608, 12288, 32), (4096, 3072, 64),
                                   (4103, 96, 32), (17550, 3072, 32), (300, 3072, 48), (4608, 12288, 48)])
def test_lowrank_down_matches_oracle(kq, M, K, r):
    """Ranks 16, 32, 64; one row to the video workload's 17550 rows; K from 96 (one
    partial chunk) to 12288; ragged last row blocks."""
    _check_lowrank(kq, M, K, r)


def test_lowrank_down_workspace_sizes(kq):
    """No workspace (one slice), a workspace for two slices, and the full one: all within
    the same bound of the exact product."""
    import torch
    M, K, r = 300, 3072, 32
    full = kq.lowrank_down_workspace_bytes(M, K, r)
    assert full >= 2 * M * r * 4
    for nb in (0, 2 * M * r * 4, full):
        ws = torch.empty((nb,), dtype=torch.uint8, device="cuda") if nb else None
        _check_lowrank(kq, M, K, r, seed=5, workspace=ws)


def test_lowrank_down_repeated_calls(kq):
    """Split-K calls in a row with different shapes sharing the default workspaces: each
    call's partial sums are complete before the next call overwrites them."""
    for i, (M, K, r) in enumerate(((300, 3072, 32), (130, 12288, 32), (300, 3072, 32), (64, 5120, 16))):
        _check_lowrank(kq, M, K, r, seed=11 + i)


def test_w4a4_small_shapes(kq):
    """One k-step (K = 128), one row, N a multiple of 16 but not of the tile."""
    for M, N, K in ((1, 16, 128), (5, 48, 128), (33, 144, 256), (130, 272, 384)):
        d = _linear_case(kq, 1, 1, M, N=N, K=K, rank=32, with_mu=True)
        err = linear.rel_frobenius(d["Y"], _ref_Y(d))
        print(f"M={M} N={N} K={K}: {err:.3e}")
        assert err <= TOL


def test_w4a4_end_to_end_quality_informational(kq):
    """Not graded: the full path vs the unquantized product, with and without the transform."""
    d = _linear_case(kq, 3, 0, 128)
    exact = d["X16"].astype(np.float64) @ d["W16"].astype(np.float64).T + \
        (d["X16"].astype(np.float64) @ d["L1"].astype(np.float64).T) @ d["L2"].astype(np.float64).T
    print("end-to-end rel error (centred RPBH, MXFP4):", linear.rel_frobenius(d["Y"], exact))


def test_w2a4_linear_matches_oracle(kq):
    """Small grids (the 128 x 128 W2A4 form): SANA-like qkv and fc2 weights on 130 and 64
    tokens, N cut to 480 and 2240; oracle on every output."""
    import torch
    c = synth.CONFIGS[2]
    for layer, M, Nr in ((0, 130, 480), (2, 64, 2240)):
        _, K, N = c["layers"][layer]
        X16 = synth.activations(M, K, 2, c["sigma_mu"])
        W16, _, _ = synth.weights(K, N, 2, layer, 0)
        W16 = np.ascontiguousarray(W16[:Nr])
        xf = synth.xform_for(2, layer, K)
        dxf = _dev_xform(kq, torch, xf, K)
        xc, xs, _ = kq.transform_quantize(torch.from_numpy(X16).cuda(), dxf, fmt="lm4")
        wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="lm2", with_wbar=False)
        Y = kq.w4a4_linear_t(xc, xs, wc, ws, fmt="lm2")
        torch.cuda.synchronize()
        ref = linear.w2a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy())
        err = linear.rel_frobenius(Y.cpu().numpy(), ref)
        print(f"W2A4 layer{layer} M={M} N={Nr} K={K}: {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("layer,M,Nr", [(0, 4096, 6720), (0, 4000, 6416), (1, 4096, 5600), (2, 4096, 2240),
                                         (1, 1100, 5600)])
def test_w2a4_full_size_forms(kq, layer, M, Nr):
    """The W2A4 linear at the SANA-like sizes: the 256 x 256 form (qkv, fc2, and with M and N
    ragged against it), with its last five tile rows in half-width tiles (fc1), and in
    half-width tiles only (fewer tokens: 110 tiles of 256 x 256); oracle on sampled rows (the
    edges of the 256- and 128-row tiles) and all columns."""
    import torch
    c = synth.CONFIGS[2]
    _, K, N = c["layers"][layer]
    X16 = synth.activations(M, K, 2, c["sigma_mu"])
    W16, _, _ = synth.weights(K, N, 2, layer, 0)
    W16 = np.ascontiguousarray(W16[:Nr])
    xf = synth.xform_for(2, layer, K)
    dxf = _dev_xform(kq, torch, xf, K)
    xc, xs, _ = kq.transform_quantize(torch.from_numpy(X16).cuda(), dxf, fmt="lm4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="lm2", with_wbar=False)
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, fmt="lm2")
    torch.cuda.synchronize()
    rows = np.array(sorted(set(range(0, M, 61)) | {0, 127, 128, 255, 256, M - 129, M - 128, M - 1} - {-1}))
    rows = rows[(rows >= 0) & (rows < M)]
    ref = linear.w2a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), rows=rows)
    err = linear.rel_frobenius(Y.cpu().numpy()[rows], ref)
    print(f"W2A4 layer{layer} M={M} N={Nr} K={K}: {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("K", [2208, 2272])
def test_w2a4_half_width_tiles(kq, K):
    """The 256 x 256 W2A4 form with its last five tile rows in tiles of half the width (352
    tiles: 96 past the first round, as 220 half-width tiles), M ragged (M = 4000) and N ragged
    against both tile widths (N = 5584), with an odd number of 32-wide groups (a last step
    with one group; K = 2208 also an odd step count).  Oracle on sampled rows (both edges of
    the switch at row 2816 among them), all columns."""
    import torch
    c = synth.CONFIGS[2]
    M, N = 4000, 5584
    X16 = synth.activations(M, K, 2, c["sigma_mu"])
    W16, _, _ = synth.weights(K, c["layers"][0][2], 2, 0, 0)
    W16 = np.ascontiguousarray(W16[:N])
    xf = synth.xform_for(2, 0, K)
    dxf = _dev_xform(kq, torch, xf, K)
    xc, xs, _ = kq.transform_quantize(torch.from_numpy(X16).cuda(), dxf, fmt="lm4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="lm2", with_wbar=False)
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, fmt="lm2")
    torch.cuda.synchronize()
    rows = np.array(sorted(set(range(0, M, 97)) | {2815, 2816, 3839, 3840, M - 1}))
    ref = linear.w2a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), rows=rows)
    err = linear.rel_frobenius(Y.cpu().numpy()[rows], ref)
    print(f"W2A4 half-width tiles M={M} N={N} K={K}: {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("K", [2208, 2272])
def test_w2a4_large_form_odd_group_count(kq, K):
    """The 256 x 256 W2A4 form (one round of tiles: M = N = 4096) with an odd number of
    32-wide groups, so that its last 64-wide step holds a single group (the missing group's
    codes and scale read as zeros); K = 2208 also has an odd step count (the step after the
    two-step loop), K = 2272 an even one.  Oracle on sampled rows, all columns."""
    import torch
    c = synth.CONFIGS[2]
    M, N = 4096, 4096
    X16 = synth.activations(M, K, 2, c["sigma_mu"])
    W16, _, _ = synth.weights(K, N, 2, 0, 0)
    xf = synth.xform_for(2, 0, K)
    dxf = _dev_xform(kq, torch, xf, K)
    xc, xs, _ = kq.transform_quantize(torch.from_numpy(X16).cuda(), dxf, fmt="lm4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(np.ascontiguousarray(W16)).cuda(), dxf, fmt="lm2",
                                               with_wbar=False)
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, fmt="lm2")
    torch.cuda.synchronize()
    rows = np.array(sorted(set(range(0, M, 97)) | {0, 255, 256, M - 1}))
    ref = linear.w2a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), rows=rows)
    err = linear.rel_frobenius(Y.cpu().numpy()[rows], ref)
    print(f"W2A4 large form K={K}: {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("Nr", [2032, 2064])
def test_w2a4_forms_at_the_threshold(kq, Nr):
    """Either side of the switch to full-width tiles of the W2A4 large form on MI355X's 256
    compute units: 128 tiles of 256 x 256 (N = 2032) run as 256 half-width tiles, 144
    (N = 2064) as full ones; M and N ragged against both tile widths.  Oracle on sampled rows,
    all columns."""
    import torch
    c = synth.CONFIGS[2]
    M, K = 4000, 2240
    X16 = synth.activations(M, K, 2, c["sigma_mu"])
    W16, _, _ = synth.weights(K, c["layers"][0][2], 2, 0, 0)
    W16 = np.ascontiguousarray(W16[:Nr])
    xf = synth.xform_for(2, 0, K)
    dxf = _dev_xform(kq, torch, xf, K)
    xc, xs, _ = kq.transform_quantize(torch.from_numpy(X16).cuda(), dxf, fmt="lm4")
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="lm2", with_wbar=False)
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, fmt="lm2")
    torch.cuda.synchronize()
    rows = np.array(sorted(set(range(0, M, 89)) | {127, 128, 255, 256, M - 1}))
    ref = linear.w2a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), rows=rows)
    err = linear.rel_frobenius(Y.cpu().numpy()[rows], ref)
    print(f"W2A4 M={M} N={Nr} K={K}: {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("layer", [0, 1])
def test_w4a4_full_size_sampled(kq, layer):
    """FLUX-like qkv (M = 4608, K = 3072, N = 9216: 256 x 256 tiles only) and fc1 (N = 12288:
    its last two tile rows in tiles of half the width) at full size in the bench's launch
    configuration; oracle on sampled rows (both edges of the switch to the half-width tiles
    at row 4096 among them) and all columns."""
    d = _linear_case(kq, 3, layer, 4608)
    rows = np.array(sorted(set(range(5, 4608, 151)) | {4095, 4096, 4351, 4352, 4607}))
    ref = _ref_Y(d, rows=rows)
    err = linear.rel_frobenius(d["Y"][rows], ref)
    print(f"layer {layer} full-size sampled rel frobenius {err:.3e}")
    assert err <= TOL


def _sampled_rows(M):
    """Rows spread over the matrix plus both edges of every 256-row tile boundary near the
    ends (the large-tile kernel form works on 256 x 256 output tiles)."""
    rows = set(range(0, M, 97)) | {0, 1, 255, 256, M - 257, M - 256, M - 2, M - 1}
    return np.array(sorted(r for r in rows if 0 <= r < M))


@pytest.mark.parametrize("rank,with_mu,K", [(0, False, 1024), (16, True, 1024), (64, False, 1024), (32, True, 1024),
                                            (32, True, 1152), (0, False, 640), (16, True, 1408)])
def test_w4a4_large_tile_form_ragged(kq, rank, with_mu, K):
    """Enough 256 x 256 tiles for the large-tile (direct-to-LDS) kernel form, with M and N not
    multiples of the tile; K = 1152, 640 and 1408 leave a last group of 1, 1 and 3 k-steps of
    128 for the scale loads, whose 16-byte pieces then run into the next row (and, on the last
    row, past the end of the scales).  Oracle on sampled rows and all columns."""
    M, N = 1800, 4624
    d = _linear_case(kq, 1, 1, M, N=N, K=K, rank=rank, with_mu=with_mu)
    rows = _sampled_rows(M)
    err = linear.rel_frobenius(d["Y"][rows], _ref_Y(d, rows=rows))
    print(f"M={M} N={N} K={K} rank {rank} mu {with_mu}: {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("M,N,K", [(2041, 2032, 640), (2041, 2064, 640), (4600, 12272, 640), (4600, 11008, 1152)])
def test_w4a4_half_width_tiles(kq, M, N, K):
    """Grids with tiles of half the width (256 token rows x 128 weight rows) on MI355X's 256
    compute units: 64 and 72 tiles of 256 x 256 (N = 2032, 2064) run as half-width tiles only;
    864 tiles (N = 12272) run their last two tile rows half-width, 774 (N = 11008) their last
    one.  M ragged, N ragged against the half-width tiles too (2064 and 12272), K = 640 and
    1152 (short last scale groups), rank 32 and the rank-1 restore."""
    d = _linear_case(kq, 1, 1, M, N=N, K=K, rank=32, with_mu=True)
    rows = _sampled_rows(M)
    err = linear.rel_frobenius(d["Y"][rows], _ref_Y(d, rows=rows))
    print(f"M={M} N={N} K={K}: {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("cfg,layer", [(1, 0), (1, 3), (4, 0), (4, 1)])
def test_w4a4_full_size_other_configs(kq, cfg, layer):
    """The PixArt-like (M = 8192; qkv K = 1152, a short last scale group, and fc2 K = 4608,
    both on the large-tile form) and CogVideoX-like (M = 17550, ragged against 256-row tiles) linears
    at full size: oracle on sampled rows and all columns."""
    M = synth.CONFIGS[cfg]["M"]
    d = _linear_case(kq, cfg, layer, M)
    rows = _sampled_rows(M)
    err = linear.rel_frobenius(d["Y"][rows], _ref_Y(d, rows=rows))
    print(f"cfg{cfg} layer{layer} full size M={M}: sampled rel frobenius {err:.3e}")
    assert err <= TOL


def test_w4a4_full_size_fc2_sampled(kq):
    """FLUX-like fc2 at full size (M = 4608, K = 12288, N = 3072): oracle on sampled rows and
    all columns."""
    d = _linear_case(kq, 3, 2, 4608)
    rows = _sampled_rows(4608)
    err = linear.rel_frobenius(d["Y"][rows], _ref_Y(d, rows=rows))
    print(f"fc2 full-size sampled rel frobenius {err:.3e}")
    assert err <= TOL


def test_repeated_calls_bit_identical(kq):
    """The centred RPBH transform and the W4A4 linear at the FLUX-like qkv size give the same
    bytes on every call (no atomics, fixed summation order)."""
    import torch
    d = _linear_case(kq, 3, 0, 4608)
    X = torch.from_numpy(d["X16"]).cuda()
    dxf = _dev_xform(kq, torch, d["xf"], X.shape[1])
    ops = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (d["xc"], d["xs"], d["wc"], d["ws"], d["T"], d["L2"],
                                                                       d["mu"], d["wbar"])]
    outs, codes = [], []
    for _ in range(3):
        xc, xs, mu = kq.transform_quantize(X, dxf, fmt="mxfp4", center=True)
        codes.append((xc.cpu().numpy(), xs.cpu().numpy(), mu.cpu().numpy().view(np.uint16)))
        Y = kq.w4a4_linear_t(*ops[:4], T=ops[4], L2=ops[5], mu=ops[6], wbar=ops[7])
        outs.append(Y.cpu().numpy().view(np.uint16))
    torch.cuda.synchronize()
    for c in codes[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(codes[0], c))
    for y in outs[1:]:
        assert np.array_equal(outs[0], y)
    assert np.array_equal(outs[0], d["Y"].view(np.uint16))


# ----------------------------------------------------------------- the boundary's own forms

def test_fold_kn_layout_matches_nk(kq):
    """kq_fold_inverse_into_weights takes W [K][N] (Y = X W); its codes, scales and column
    sums are byte-identical to the [N][K] form on the same weights, and match the oracle."""
    import torch
    for cfg, layer, nrows in ((3, 0, 200), (4, 0, 96), (1, 3, 80)):
        c = synth.CONFIGS[cfg]
        _, K, N = c["layers"][layer]
        W16, _, _ = synth.weights(K, N, cfg, layer, 0)
        W16 = np.ascontiguousarray(W16[:nrows])                 # [N][K]
        xf = synth.xform_for(cfg, layer, K)
        dxf = _dev_xform(kq, torch, xf, K)
        a = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="mxfp4")
        b = kq.fold_inverse_into_weights(torch.from_numpy(np.ascontiguousarray(W16.T)).cuda(), dxf, fmt="mxfp4")
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v)
        _wbar_check(W16, b[2].cpu().numpy())
    # and the 2-bit weight format
    c = synth.CONFIGS[2]
    _, K, N = c["layers"][0]
    W16 = np.ascontiguousarray(synth.weights(K, N, 2, 0, 0)[0][:64])
    dxf = _dev_xform(kq, torch, synth.xform_for(2, 0, K), K)
    a = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="lm2")
    b = kq.fold_inverse_into_weights(torch.from_numpy(np.ascontiguousarray(W16.T)).cuda(), dxf, fmt="lm2")
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def _x_form_case(kq, cfg, layer, M, r, with_mu, K=None, N=None):
    """Operands for the linear that runs its own down-projection: the activation path on
    the GPU, weights folded from [K][N]."""
    import torch
    c = synth.CONFIGS[cfg]
    _, K0, N0 = c["layers"][layer]
    K = K0 if K is None else K
    N = N0 if N is None else N
    X16 = synth.activations(M, K, cfg, c["sigma_mu"], c["frames"])
    W16, L1, L2 = synth.weights(K, N, cfg, layer, max(r, 1))
    xf = synth.xform_for(cfg, layer, K) if K == K0 else {"kind": "kron", "A": synth.kron_factors(cfg, layer)[0],
                                                          "B": synth.kron_factors(cfg, layer)[1]}
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, mu = kq.transform_quantize(X, dxf, fmt="mxfp4", center=with_mu)
    wc, ws, wbar = kq.fold_inverse_into_weights(torch.from_numpy(np.ascontiguousarray(W16.T)).cuda(), dxf)
    L1d = torch.from_numpy(np.ascontiguousarray(L1[:r])).cuda() if r else None
    L2d = torch.from_numpy(np.ascontiguousarray(L2[:, :r])).cuda() if r else None
    return dict(X16=X16, X=X, L1=L1[:r] if r else None, L2=np.ascontiguousarray(L2[:, :r]) if r else None,
                L1d=L1d, L2d=L2d, xc=xc, xs=xs, wc=wc, ws=ws, mu=mu, wbar=wbar if with_mu else None)


@pytest.mark.parametrize("cfg,layer,M,r,with_mu", [(3, 0, 150, 32, True), (3, 2, 70, 48, True), (1, 1, 201, 16, False),
                                                     (4, 0, 97, 64, False), (0, 0, 256, 0, False), (1, 3, 77, 48, False)])
def test_w4a4_linear_x_form_matches_oracle(kq, cfg, layer, M, r, with_mu):
    """kq_w4a4_linear with X, L1, L2 and a workspace: the down-projection runs inside the
    call; every rank the boundary takes (0, 16, 32, 48, 64); against the oracle within
    2e-3, and byte-identical to the down-projection call followed by the T form."""
    import torch
    d = _x_form_case(kq, cfg, layer, M, r, with_mu)
    Y = kq.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"], X=d["X"] if r else None, L1=d["L1d"], L2=d["L2d"],
                       mu=d["mu"], wbar=d["wbar"])
    T = kq.lowrank_down(d["X"], d["L1d"]) if r else None
    Y2 = kq.w4a4_linear_t(d["xc"], d["xs"], d["wc"], d["ws"], T=T, L2=d["L2d"], mu=d["mu"], wbar=d["wbar"])
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    ref = linear.w4a4_linear(d["xc"].cpu().numpy(), d["xs"].cpu().numpy(), d["wc"].cpu().numpy(),
                             d["ws"].cpu().numpy(), d["X16"] if r else None, d["L1"], d["L2"],
                             None if d["mu"] is None else d["mu"].cpu().numpy(),
                             None if d["wbar"] is None else d["wbar"].cpu().numpy())
    err = linear.rel_frobenius(Y.cpu().numpy(), ref)
    print(f"x-form cfg{cfg} layer{layer} M={M} r={r} mu={with_mu}: {err:.3e}")
    assert err <= TOL


def test_w4a4_linear_x_form_full_size_sampled(kq):
    """The FLUX-like qkv at full size through the boundary's own form (M = 4608, K = 3072,
    N = 9216, centred, rank 32), in the bench's launch configuration; sampled rows."""
    import torch
    d = _x_form_case(kq, 3, 0, 4608, 32, True)
    ws = torch.empty((kq.w4a4_linear_workspace_bytes(4608, 32),), dtype=torch.uint8, device="cuda")
    Y = kq.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"], X=d["X"], L1=d["L1d"], L2=d["L2d"], mu=d["mu"],
                       wbar=d["wbar"], workspace=ws)
    torch.cuda.synchronize()
    rows = _sampled_rows(4608)
    ref = linear.w4a4_linear(d["xc"].cpu().numpy(), d["xs"].cpu().numpy(), d["wc"].cpu().numpy(),
                             d["ws"].cpu().numpy(), d["X16"], d["L1"], d["L2"], d["mu"].cpu().numpy(),
                             d["wbar"].cpu().numpy(), rows=rows)
    err = linear.rel_frobenius(Y.cpu().numpy()[rows], ref)
    print(f"x-form full size sampled: {err:.3e}")
    assert err <= TOL


def test_w4a4_linear_x_form_workspace_errors(kq):
    """A workspace smaller than kq_w4a4_linear_workspace_bytes is refused before anything is
    launched (KQ_ERR_WORKSPACE), and a sufficient one works."""
    import torch
    d = _x_form_case(kq, 3, 0, 64, 32, False)
    need = kq.w4a4_linear_workspace_bytes(64, 32)
    small = torch.empty((need - 256,), dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"], X=d["X"], L1=d["L1d"], L2=d["L2d"], workspace=small)
    assert e.value.status == 7
    ok = torch.empty((need,), dtype=torch.uint8, device="cuda")
    kq.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"], X=d["X"], L1=d["L1d"], L2=d["L2d"], workspace=ok)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1801, 1807])
def test_w4a4_large_tile_ragged_means(kq, M):
    """The large-tile form with the rank-1 restore when the last 256-row tile holds a number
    of rows that is not a multiple of 8 (odd, too): the means of the last rows reach the
    epilogue; also with mu given as an offset view (2-byte aligned, not 16)."""
    import torch
    N, K = 4624, 1024
    d = _linear_case(kq, 1, 1, M, N=N, K=K, rank=32, with_mu=True)
    rows = np.array(sorted(set(_sampled_rows(M)) | set(range(M - 9, M))))
    err = linear.rel_frobenius(d["Y"][rows], _ref_Y(d, rows=rows))
    print(f"M={M}: {err:.3e}")
    assert err <= TOL
    # the same call with mu at an odd fp16 offset inside a larger buffer
    buf = torch.zeros((M + 1,), dtype=torch.float16, device="cuda")
    buf[1:] = torch.from_numpy(d["mu"]).cuda()
    mu_view = buf[1:]
    assert mu_view.data_ptr() % 16 != 0
    ops = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (d["xc"], d["xs"], d["wc"], d["ws"], d["T"],
                                                                       d["L2"], d["wbar"])]
    Y2 = kq.w4a4_linear_t(*ops[:4], T=ops[4], L2=ops[5], mu=mu_view, wbar=ops[6])
    torch.cuda.synchronize()
    assert np.array_equal(Y2.cpu().numpy().view(np.uint16), d["Y"].view(np.uint16))


def test_calls_on_a_non_current_stream(kq):
    """Calls given another stream than torch's current one: their internally allocated
    workspaces and outputs are kept alive for that stream (record_stream), and the
    results equal those of the same calls on the current stream."""
    import torch
    M, K, r = 300, 3072, 32
    X16 = synth.activations(M, K, 7, 2.0)
    _, L1, _ = synth.weights(K, 16, 7, 0, r)
    X = torch.from_numpy(X16).cuda()
    L1d = torch.from_numpy(L1).cuda()
    ref = kq.lowrank_down(X, L1d)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(4):
        outs.append(kq.lowrank_down(X, L1d, stream=s))
        # churn torch's allocator on the current stream meanwhile
        junk = [torch.empty((1 << 20,), dtype=torch.uint8, device="cuda").fill_(7) for _ in range(8)]
        del junk
    s.synchronize()
    torch.cuda.synchronize()
    for t in outs:
        assert torch.equal(t, ref)
