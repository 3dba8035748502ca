"""GPU parity of the offline rank-r extraction (kq_svd_lowrank) against the oracle's LAPACK
SVD, on weights whose leading directions stand out (planted low-rank part over a Gaussian
bulk).  The factors are unique only up to signs, so the unique quantities are compared:
the singular values, the rank-r product L2 L1, the residual's norm, and the residual's
definition R = fp16(W - L2 L1) on the kernel's own factors."""

import numpy as np
import pytest

import synth
from oracle import linear, pipeline, svd, ties
from tests.test_gpu_transform import _dev_xform

pytestmark = pytest.mark.gpu


def _run(kq, Wt16, r, l, iters, seed):
    import torch
    W = torch.from_numpy(Wt16).cuda()
    om = torch.from_numpy(synth.gaussian_block(Wt16.shape[1], l, seed)).cuda()
    L1, L2, R, sg = kq.svd_lowrank(W, r, om, iters=iters)
    torch.cuda.synchronize()
    return L1.cpu().numpy(), L2.cpu().numpy(), R.cpu().numpy(), sg.cpu().numpy()


def _check_residual(Wt16, L1, L2, R):
    """R = fp16(Wt - L2 L1) on these factors: within half an fp16 step of the float64
    value plus the float32 bound of the r-term product (one step at a rounding tie)."""
    P = L2.astype(np.float64) @ L1.astype(np.float64)
    ref = Wt16.astype(np.float64) - P
    bound = ties.gamma_tau(L1.shape[0] + 2, np.abs(L2.astype(np.float64)) @ np.abs(L1.astype(np.float64)))
    step = np.maximum(np.abs(ref), 2.0 ** -14) * 2.0 ** -10
    assert np.all(np.abs(R.astype(np.float64) - ref) <= step + bound)


@pytest.mark.parametrize("N,K,r,l,iters", [(160, 1152, 16, 32, 4), (1536, 3072, 32, 48, 4), (384, 12288, 32, 48, 3),
                                           (64, 96, 16, 24, 4), (512, 3072, 64, 80, 4)])
def test_svd_lowrank_matches_oracle(kq, N, K, r, l, iters):
    Wt16 = synth.planted_lowrank_weights(K, N, 30, 0, r)
    L1, L2, R, sg = _run(kq, Wt16, r, l, iters, 31)
    ref = svd.svd_lowrank(Wt16, r)
    s = ref["s"][:r]
    assert np.all(np.abs(sg - s) <= 1e-4 * s[0]), np.max(np.abs(sg - s) / s[0])
    L1o, L2o, _ = svd.svd_lowrank_f64(Wt16, r)
    Po = L2o @ L1o
    Pg = L2.astype(np.float64) @ L1.astype(np.float64)
    err = linear.rel_frobenius(Pg, Po)
    print(f"svd N={N} K={K} r={r}: sigma max rel err {np.max(np.abs(sg - s)) / s[0]:.2e}, product rel {err:.2e}")
    assert err <= 2e-3
    _check_residual(Wt16, L1, L2, R)
    ng, no = np.linalg.norm(R.astype(np.float64)), np.linalg.norm(ref["R64"])
    assert abs(ng - no) <= 1e-2 * no, (ng, no)


def test_svd_lowrank_without_power_steps(kq):
    """iters = 0 (one product and one projection): a coarser subspace, but the residual is
    still exactly W minus the kernel's own factors."""
    Wt16 = synth.planted_lowrank_weights(1152, 256, 32, 0, 16)
    L1, L2, R, sg = _run(kq, Wt16, 16, 32, 0, 33)
    _check_residual(Wt16, L1, L2, R)
    assert np.all(np.isfinite(sg)) and np.all(np.diff(sg) <= 0)


def test_svd_then_fold_and_linear(kq):
    """The whole SVDQuant-style layer: the residual is folded and quantized, the extracted
    factors form the 16-bit branch; against the exact X W, the 4-bit error is smaller than
    quantizing all of W with a random branch of the same rank."""
    import torch
    M, K, N, r = 256, 3072, 512, 32
    X16 = synth.activations(M, K, 34, 2.0)
    Wt16 = synth.planted_lowrank_weights(K, N, 34, 0, r)
    L1, L2, R, _ = _run(kq, Wt16, r, 48, 4, 35)
    A, B = synth.kron_factors(34, 0)
    xf = {"kind": "kron", "A": A, "B": B}
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, _, T = kq.transform_quantize_lowrank(X, dxf, torch.from_numpy(L1).cuda())
    wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(R).cuda(), dxf, fmt="mxfp4")
    Y = kq.w4a4_linear_t(xc, xs, wc, ws, T=T, L2=torch.from_numpy(np.ascontiguousarray(L2)).cuda())
    torch.cuda.synchronize()
    ref = linear.w4a4_linear(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), X16, L1, L2,
                             None, None)
    assert linear.rel_frobenius(Y.cpu().numpy(), ref) <= 2e-3
    exact = X16.astype(np.float64) @ Wt16.astype(np.float64).T
    e_svd = linear.rel_frobenius(Y.cpu().numpy(), exact)
    # without extraction: all of W quantized, no branch
    wc2, ws2, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(Wt16).cuda(), dxf, fmt="mxfp4")
    Y2 = kq.w4a4_linear_t(xc, xs, wc2, ws2)
    torch.cuda.synchronize()
    e_plain = linear.rel_frobenius(Y2.cpu().numpy(), exact)
    print(f"4-bit error against exact X W: with extraction {e_svd:.3e}, without {e_plain:.3e}")
    assert e_svd < e_plain


def test_svd_rejects_bad_arguments(kq):
    import torch
    W = torch.zeros((64, 96), dtype=torch.float16, device="cuda")
    with pytest.raises(kq.KQError):
        kq.svd_lowrank(W, 16, torch.zeros((96, 16), dtype=torch.float32, device="cuda"))    # l == r
    with pytest.raises(kq.KQError):
        kq.svd_lowrank(W, 16, torch.zeros((96, 97), dtype=torch.float32, device="cuda"))    # l > 96
    with pytest.raises(kq.KQError):
        kq.svd_lowrank(W, 16, torch.zeros((96, 24), dtype=torch.float32, device="cuda"), iters=17)
