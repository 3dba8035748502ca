"""The allocation-free linear (kq_w4a4_linear_noalloc), called through the C ABI: its
output equals the workspace form's (kq_w4a4_linear) on the same operands, on two calls in
a row with the second one smaller (the library's scratch array keeps the first call's
contents), and the first call is checked against the oracle to the linear's 2e-3 bar."""

import ctypes

import numpy as np
import pytest

import synth
from oracle import linear
from tests.test_gpu_linear import _dev_xform

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _operands(kq, cfg, layer, M, r, center, N=None):
    import torch
    c = synth.CONFIGS[cfg]
    _, K, N0 = c["layers"][layer]
    N = N0 if N is None else N
    X16 = synth.activations(M, K, cfg, c["sigma_mu"], c["frames"])
    W16, L1, L2 = synth.weights(K, N, cfg, layer, r)
    xf = synth.xform_for(cfg, layer, K)
    dxf = _dev_xform(kq, torch, xf, K)
    X = torch.from_numpy(X16).cuda()
    xc, xs, mu = kq.transform_quantize(X, dxf, fmt="mxfp4", center=center)
    wc, ws, wbar = kq.fold_inverse_into_weights(torch.from_numpy(np.ascontiguousarray(W16.T)).cuda(), dxf)
    dev = (lambda a: None if a is None else torch.from_numpy(a).cuda())
    return dict(X16=X16, X=X, L1=L1, L2=L2, L1d=dev(L1), L2d=dev(L2),
                xc=xc, xs=xs, wc=wc, ws=ws, mu=mu, wbar=wbar if center else None, M=M, K=K, N=N, r=r)


def _noalloc(kq, d):
    """One call of kq_w4a4_linear_noalloc through ctypes, on torch's current stream."""
    import torch
    Y = torch.empty((d["M"], d["N"]), dtype=torch.float16, device="cuda")
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    s = kq.load().kq_w4a4_linear_noalloc(0, p(d["xc"]), p(d["xs"]), d["M"], d["K"], p(d["wc"]), p(d["ws"]), d["N"],
                                         p(d["X"]), p(d["L1d"]), p(d["L2d"]), d["r"], p(d["mu"]), p(d["wbar"]),
                                         p(Y), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert s == 0, kq.status_str(s)
    return Y


def _with_workspace(kq, d):
    return kq.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"], X=d["X"], L1=d["L1d"], L2=d["L2d"], mu=d["mu"],
                          wbar=d["wbar"])


def test_noalloc_linear_two_calls_second_smaller(kq):
    import torch
    big = _operands(kq, 3, 0, 4608, 32, True)              # FLUX-like qkv, full size, centred
    small = _operands(kq, 1, 1, 300, 16, False, N=1152)    # PixArt-like proj, fewer rows, lower rank
    y_big = _noalloc(kq, big)
    y_small = _noalloc(kq, small)
    ref_big = _with_workspace(kq, big)
    ref_small = _with_workspace(kq, small)
    torch.cuda.synchronize()
    for got, ref, name in ((y_big, ref_big, "first (M=4608, r=32)"), (y_small, ref_small, "second (M=300, r=16)")):
        err = linear.rel_frobenius(got.cpu().numpy(), ref.cpu().numpy().astype(np.float64))
        same = torch.equal(got, ref)
        print(f"no-alloc {name}: identical to the workspace form: {same}; rel frobenius {err:.3e}")
        assert err <= TOL
        assert same          # same K split, same arithmetic
    # the first call against the oracle on sampled rows
    rows = np.arange(3, 4608, 211)
    o = linear.w4a4_linear(big["xc"].cpu().numpy(), big["xs"].cpu().numpy(), big["wc"].cpu().numpy(),
                           big["ws"].cpu().numpy(), big["X16"], big["L1"], big["L2"], big["mu"].cpu().numpy(),
                           big["wbar"].cpu().numpy(), rows=rows)
    err = linear.rel_frobenius(y_big.cpu().numpy()[rows], o)
    print(f"no-alloc first call vs oracle (sampled rows): {err:.3e}")
    assert err <= TOL


def test_noalloc_linear_without_branch(kq):
    """r = 0: no down-projection, nothing in the scratch; equal to the workspace form."""
    import torch
    d = _operands(kq, 0, 0, 256, 0, False)
    d["L1d"] = d["L2d"] = d["X"] = None
    y = _noalloc(kq, d)
    ref = kq.w4a4_linear(d["xc"], d["xs"], d["wc"], d["ws"])
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
