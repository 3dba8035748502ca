"""GPU parity of the fused pass (kq_transform_quantize_lowrank): one read of X gives the
MXFP4 codes of the block-transformed activations and the low-rank down-projection T.

Both outputs are checked against the oracle (codes with the tie rule, T against the fp64
product within its float32 accumulation bound) and, bit for bit, against the two separate
calls, which run the same arithmetic."""

import numpy as np
import pytest

import synth
from oracle import linear, ties
from tests import gpu_util
from tests.test_gpu_transform import _dev_xform

pytestmark = pytest.mark.gpu


def _xf(kind, seed, K):
    if kind == "kron":
        A, B = synth.kron_factors(seed, 0)
        return {"kind": "kron", "A": A, "B": B}
    if kind == "dense":
        return {"kind": "dense", "P": synth.dense_block(seed, 0)}
    return {"kind": "none"}


def _run(kq, X16, L1, xf):
    import torch
    X = torch.from_numpy(X16).cuda()
    L = torch.from_numpy(np.ascontiguousarray(L1)).cuda()
    dxf = _dev_xform(kq, torch, xf, X16.shape[1])
    c, s, _, T = kq.transform_quantize_lowrank(X, dxf, L)
    c2, s2, _ = kq.transform_quantize(X, dxf, fmt="mxfp4")
    T2 = kq.lowrank_down(X, L)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (c, s, T, c2, s2, T2)]


def _check_T(X16, L1, T, rows=None):
    """Within one fp16 rounding of the exact product plus the float32 accumulation bound
    (the rule of the separate down-projection's test)."""
    K = X16.shape[1]
    X = X16.astype(np.float64) if rows is None else X16[rows].astype(np.float64)
    exact = X @ L1.astype(np.float64).T
    bound = np.abs(X) @ np.abs(L1.astype(np.float64)).T
    got = (T if rows is None else T[rows]).astype(np.float64)
    assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -11 + ties.gamma_tau(K // 8 + 16, bound) + 2.0 ** -24)


@pytest.mark.parametrize("kind", ["kron", "dense", "none"])
@pytest.mark.parametrize("M,K,r", [(300, 1152, 32), (203, 160, 16), (7, 96, 64), (1000, 12288, 32), (64, 3072, 16),
                                   (1, 32, 16), (65, 32, 32)])
def test_fused_matches_oracle_and_separate_calls(kq, kind, M, K, r):
    X16 = synth.activations(M, K, 21, 2.0)
    _, L1, _ = synth.weights(K, 64, 21, 0, r)
    xf = _xf(kind, 21, K)
    c, s, T, c2, s2, T2 = _run(kq, X16, L1, xf)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    assert np.array_equal(T.view(np.uint16), T2.view(np.uint16))
    y, tau, _ = gpu_util.oracle_activation_reference(X16, xf, False)
    gpu_util.assert_mx_parity(c, s, y, tau, label=f"fused {kind} M={M} K={K} r={r}")
    _check_T(X16, L1, T)


def test_fused_full_size_sampled_rows(kq):
    """The FLUX-like width at full M (4608 x 3072, rank 32), Kronecker factors: sampled rows
    against the oracle, all rows against the separate calls."""
    M, K, r = 4608, 3072, 32
    X16 = synth.activations(M, K, 22, 4.0)
    _, L1, _ = synth.weights(K, 64, 22, 0, r)
    xf = _xf("kron", 22, K)
    c, s, T, c2, s2, T2 = _run(kq, X16, L1, xf)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    assert np.array_equal(T.view(np.uint16), T2.view(np.uint16))
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    y, tau, _ = gpu_util.oracle_activation_reference(X16[rows], xf, False)
    gpu_util.assert_mx_parity(c[rows], s[rows], y, tau, label="fused full sampled")
    _check_T(X16, L1, T, rows)


def test_fused_linear(kq):
    """The whole layer from the fused pass: Y = Xq Wq^T + T L2^T against the oracle on the
    kernel's own packed operands."""
    import torch
    M, K, N, r = 300, 3072, 384, 32
    X16 = synth.activations(M, K, 23, 2.0)
    W16, L1, L2 = synth.weights(K, N, 23, 0, r)
    xf = _xf("kron", 23, K)
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, _, T = kq.transform_quantize_lowrank(X, dxf, torch.from_numpy(L1).cuda())
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W16).cuda(), dxf, fmt="mxfp4")
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=torch.from_numpy(np.ascontiguousarray(L2)).cuda())
    torch.cuda.synchronize()
    ref = linear.w4a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), X16, L1, L2,
                             None, None)
    err = linear.rel_frobenius(Y.cpu().numpy(), ref)
    print(f"fused linear rel frobenius {err:.3e}")
    assert err <= 2e-3


def test_fused_rejects_unsupported(kq):
    """Centring is offered with RPBH only; no power-of-two scaling; no per-block factors."""
    import torch
    X = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    L = torch.zeros((16, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(kq.KQError):
        kq.transform_quantize_lowrank(X, kq.Xform.none(64), L, center=True)
    with pytest.raises(kq.KQError):
        kq.transform_quantize_lowrank(X, kq.Xform.none(64).with_pts(torch.zeros(64, dtype=torch.int8, device="cuda")),
                                      L)
    AB = torch.zeros((2, 80), dtype=torch.float32, device="cuda")
    with pytest.raises(kq.KQError):
        kq.transform_quantize_lowrank(X, kq.Xform.kron_blocks(AB, 64), L)


# ------------------------------------------------------------------ RPBH with centring

def _rpbh_case(kq, M, K, r, center, seed=26, sigma=4.0):
    import torch
    X16 = synth.activations(M, K, seed, sigma)
    _, L1, _ = synth.weights(K, 64, seed, 0, r)
    perm, sign = synth.rpbh_params(K, seed, 0)
    xf = {"kind": "rpbh", "perm": perm, "sign": sign}
    X = torch.from_numpy(X16).cuda()
    L = torch.from_numpy(np.ascontiguousarray(L1)).cuda()
    dxf = _dev_xform(kq, torch, xf, K)
    c, s, mu, T = kq.transform_quantize_lowrank(X, dxf, L, center=center)
    torch.cuda.synchronize()
    return X16, L1, xf, c.cpu().numpy(), s.cpu().numpy(), None if mu is None else mu.cpu().numpy(), T.cpu().numpy()


def _check_rpbh(X16, L1, xf, c, s, mu, T, center, label, rows=None):
    sel = slice(None) if rows is None else rows
    Xs = X16[sel]
    if center:
        gpu_util.check_mu(Xs, mu[sel])
    y, tau, _ = gpu_util.oracle_activation_reference(Xs, xf, center, mu_gpu=None if mu is None else mu[sel])
    gpu_util.assert_mx_parity(c[sel], s[sel], y, tau, label=label)
    _check_T(X16, L1, T, rows)


@pytest.mark.parametrize("center", [True, False])
@pytest.mark.parametrize("M,K,r", [(203, 3072, 32), (97, 3072, 16), (1, 32, 32), (3, 2240, 32), (130, 6144, 16),
                                   (67, 1152, 32), (77, 6144, 32), (41, 12288, 32)])
def test_fused_rpbh_matches_oracle(kq, center, M, K, r):
    """RPBH (centred or not) + MXFP4 + the down-projection in one call (the row-staged
    transform, then the split-K projection); ragged row groups, one row, one block per
    row, K up to 12288.  Codes, scales and means against the oracle with the tie rules, T
    within the float32 bound of the exact product."""
    X16, L1, xf, c, s, mu, T = _rpbh_case(kq, M, K, r, center)
    _check_rpbh(X16, L1, xf, c, s, mu, T, center, f"fused rpbh M={M} K={K} r={r} center={center}")


def test_fused_rpbh_full_size_sampled(kq):
    """The FLUX-like qkv input at full size (M = 4608, K = 3072, rank 32, centred), in the
    launch configuration the bench times; oracle on sampled rows, T on the same rows."""
    M, K, r = 4608, 3072, 32
    X16, L1, xf, c, s, mu, T = _rpbh_case(kq, M, K, r, True, seed=3)
    rows = np.unique(np.concatenate([np.arange(0, M, 89), [M - 4, M - 3, M - 2, M - 1]]))
    _check_rpbh(X16, L1, xf, c, s, mu, T, True, "fused rpbh full size sampled", rows=rows)


def test_fused_rpbh_agrees_with_separate_calls(kq):
    """The call runs the same kernels as the two separate calls (transform, then
    down-projection with a workspace of the same size): codes, scales, means and T are
    bit-identical to theirs."""
    import torch
    M, K, r = 800, 3072, 32
    X16, L1, xf, c, s, mu, T = _rpbh_case(kq, M, K, r, True, seed=27)
    X = torch.from_numpy(X16).cuda()
    dxf = _dev_xform(kq, torch, xf, K)
    c2, s2, mu2 = kq.transform_quantize(X, dxf, fmt="mxfp4", center=True)
    T2 = kq.lowrank_down(X, torch.from_numpy(np.ascontiguousarray(L1)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(c, c2.cpu().numpy())
    assert np.array_equal(s, s2.cpu().numpy())
    assert np.array_equal(mu.view(np.uint16), mu2.cpu().numpy().view(np.uint16))
    assert np.array_equal(T.view(np.uint16), T2.cpu().numpy().view(np.uint16))


def test_fused_rpbh_linear(kq):
    """The FLUX-like layer from the fused pass: Y = Xq Wq^T + T L2^T + mu wbar^T against the
    oracle on the kernel's own packed operands."""
    import torch
    M, K, N, r = 300, 3072, 384, 32
    X16 = synth.activations(M, K, 3, 4.0)
    W16, L1, L2 = synth.weights(K, N, 3, 0, r)
    perm, sign = synth.rpbh_params(K, 3, 0)
    xf = {"kind": "rpbh", "perm": perm, "sign": sign}
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, mu, T = kq.transform_quantize_lowrank(X, dxf, torch.from_numpy(L1).cuda(), center=True)
    wc, ws, wbar = kq.fold_inverse_into_weights(torch.from_numpy(np.ascontiguousarray(W16.T)).cuda(), dxf)
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=torch.from_numpy(np.ascontiguousarray(L2)).cuda(), mu=mu, wbar=wbar)
    torch.cuda.synchronize()
    ref = linear.w4a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), X16, L1, L2,
                             mu.cpu().numpy(), wbar.cpu().numpy())
    err = linear.rel_frobenius(Y.cpu().numpy(), ref)
    print(f"fused rpbh linear rel frobenius {err:.3e}")
    assert err <= 2e-3
