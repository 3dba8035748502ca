"""GPU parity of the online activation path (transform + quantize) against the oracle.

Codes and E8M0 scales must match the float64 oracle except at logged float32 rounding
ties (mismatch fraction <= 1e-4, zero non-tie mismatches); fp16 means must match except
at rounding ties; per-token Lloyd-Max scales within their float32 error bound.
"""

import numpy as np
import pytest

import synth
from oracle import lloyd_max, mxfp4, pipeline, ties
from tests import gpu_util

pytestmark = pytest.mark.gpu


def _dev_xform(kq, torch, xf, K):
    if xf["kind"] == "kron":
        d = kq.Xform.kron(xf["A"], xf["B"], K)
    elif xf["kind"] == "rpbh":
        d = kq.Xform.rpbh(torch.from_numpy(np.ascontiguousarray(xf["perm"], dtype=np.int32)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(xf["sign"], dtype=np.int8)).cuda())
    elif xf["kind"] == "dense":
        d = kq.Xform.dense(torch.from_numpy(np.ascontiguousarray(xf["P"], dtype=np.float32)).cuda(), K)
    elif xf["kind"] == "kron_blocks":
        d = kq.Xform.kron_blocks(torch.from_numpy(kq.Xform.pack_block_factors(xf["A"], xf["B"])).cuda(), K)
    else:
        d = kq.Xform.none(K)
    if xf.get("pts") is not None:
        d = d.with_pts(torch.from_numpy(np.ascontiguousarray(xf["pts"], dtype=np.int8)).cuda())
    return d


def _run(kq, X16, xf, fmt, center):
    import torch
    X = torch.from_numpy(X16).cuda()
    dxf = _dev_xform(kq, torch, xf, X16.shape[1])
    codes, scales, mu = kq.transform_quantize(X, dxf, fmt=fmt, center=center)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), None if mu is None else mu.cpu().numpy()


def _mx_check(kq, X16, xf, center, label):
    codes, scales, mu = _run(kq, X16, xf, "mxfp4", center)
    if center:
        gpu_util.check_mu(X16, mu)
    y, tau, _ = gpu_util.oracle_activation_reference(X16, xf, center, mu_gpu=mu)
    return gpu_util.assert_mx_parity(codes, scales, y, tau, label=label)


# (config, layer, rows): rows chosen to span several waves/tiles with a ragged tail
CASES = [(0, 0, 256), (1, 0, 301), (1, 3, 97), (3, 0, 203), (3, 2, 67), (4, 0, 333), (4, 1, 129)]


@pytest.mark.parametrize("cfg,layer,rows", CASES)
def test_mxfp4_codes_match_oracle(kq, cfg, layer, rows):
    c = synth.CONFIGS[cfg]
    _, K, _ = c["layers"][layer]
    X16 = synth.activations(rows, K, cfg, c["sigma_mu"], c["frames"])
    xf = synth.xform_for(cfg, layer, K)
    _mx_check(kq, X16, xf, c["center"], f"cfg{cfg} layer{layer} M={rows} K={K}")


@pytest.mark.parametrize("kind,center", [("kron", True), ("rpbh", False), ("none", False), ("none", True)])
def test_mxfp4_other_combinations(kq, kind, center):
    K, rows = 1152, 150
    X16 = synth.activations(rows, K, 11, 3.0)
    if kind == "kron":
        A, B = synth.kron_factors(11, 0)
        xf = {"kind": "kron", "A": A, "B": B}
    elif kind == "rpbh":
        perm, sign = synth.rpbh_params(K, 11, 0)
        xf = {"kind": "rpbh", "perm": perm, "sign": sign}
    else:
        xf = {"kind": "none"}
    _mx_check(kq, X16, xf, center, f"{kind} center={center}")


@pytest.mark.parametrize("K,rows", [(3072, 203), (1152, 150), (96, 7)])
def test_mxfp4_dense_block_matches_oracle(kq, K, rows):
    """A dense learned 32x32 P (KroQuant section 01's unfactored transform) on the
    streaming matrix-core path."""
    X16 = synth.activations(rows, K, 12, 2.0)
    xf = {"kind": "dense", "P": synth.dense_block(12, 0)}
    _mx_check(kq, X16, xf, False, f"dense K={K} M={rows}")


def test_dense_block_rejects_unsupported(kq):
    """Centring and the Lloyd-Max format are not offered with a dense P."""
    import torch
    X = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    P = torch.eye(32, dtype=torch.float32, device="cuda")
    for fmt, center in (("mxfp4", True), ("lm4", False)):
        with pytest.raises(kq.KQError):
            kq.transform_quantize(X, kq.Xform.dense(P, 64), fmt=fmt, center=center)


@pytest.mark.parametrize("kind", ["kron", "dense", "none"])
@pytest.mark.parametrize("K,rows,which", [(3072, 203, "outliers"), (1152, 150, "random"), (96, 7, "random"),
                                          (12288, 37, "outliers"), (32, 1, "random")])
def test_mxfp4_pts_matches_oracle(kq, kind, K, rows, which):
    """DMQ's power-of-two channel scaling ahead of the block transform: exponents 6 on the
    planted outlier channels, or uniform 0..15 on every channel (many fp16 subnormal
    results, rounded to nearest even on both sides)."""
    X16 = synth.activations(rows, K, 13, 2.0)
    pts = synth.pts_exponents(K, synth.outlier_channels(rows, K, 13, 2.0)) if which == "outliers" \
        else synth.pts_exponents(K, seed=K)
    xf = {"kind": kind, "pts": pts}
    if kind == "kron":
        xf["A"], xf["B"] = synth.kron_factors(13, 0)
    if kind == "dense":
        xf["P"] = synth.dense_block(13, 0)
    _mx_check(kq, X16, xf, False, f"pts {which} {kind} K={K} M={rows}")


@pytest.mark.parametrize("K,rows,pts", [(3072, 203, False), (1152, 150, False), (96, 7, False), (12288, 37, False),
                                        (64, 1, False), (32, 17, False), (1152, 150, True), (3072, 48, True),
                                        (32, 3, True)])
def test_mxfp4_kron_blocks_matches_oracle(kq, K, rows, pts):
    """Per-block Kronecker factors (one (A_b, B_b) per block index) on their matrix-core
    kernel (pairs of block indices per step, odd index counts included); ragged row
    counts, one row, and power-of-two channel scaling ahead of it (random exponents
    0..15)."""
    X16 = synth.activations(rows, K, 17, 2.0)
    A, B = synth.kron_block_factors(17, 0, K // 32)
    xf = {"kind": "kron_blocks", "A": A, "B": B}
    if pts:
        xf["pts"] = synth.pts_exponents(K, seed=K + 1)
    _mx_check(kq, X16, xf, False, f"kron_blocks K={K} M={rows} pts={pts}")


def test_kron_blocks_full_size_sampled_rows(kq):
    """The FLUX-like width at full M (4608 x 12288): codes of sampled rows against the
    oracle, in the launch the bench times."""
    M, K = 4608, 12288
    X16 = synth.activations(M, K, 18, 4.0)
    A, B = synth.kron_block_factors(18, 0, K // 32)
    xf = {"kind": "kron_blocks", "A": A, "B": B}
    codes, scales, _ = _run(kq, X16, xf, "mxfp4", False)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    y, tau, _ = gpu_util.oracle_activation_reference(X16[rows], xf, False)
    gpu_util.assert_mx_parity(codes[rows], scales[rows], y, tau, label=f"kron_blocks full sampled {len(rows)}")


def test_kron_blocks_rejects_unsupported(kq):
    """Per-block factors are offered on the MXFP4 path without centring only."""
    import torch
    X = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    AB = torch.zeros((2, 80), dtype=torch.float32, device="cuda")
    for fmt, center in (("mxfp4", True), ("lm4", False)):
        with pytest.raises(kq.KQError):
            kq.transform_quantize(X, kq.Xform.kron_blocks(AB, 64), fmt=fmt, center=center)
    with pytest.raises(ValueError):
        kq.Xform.kron_blocks(torch.zeros((3, 80), dtype=torch.float32, device="cuda"), 64)


def test_pts_rejects_unsupported(kq):
    """Power-of-two scaling is offered on the streaming MXFP4 path only."""
    import torch
    X = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    e = torch.zeros(64, dtype=torch.int8, device="cuda")
    for fmt, center in (("mxfp4", True), ("lm4", False)):
        with pytest.raises(kq.KQError):
            kq.transform_quantize(X, kq.Xform.none(64).with_pts(e), fmt=fmt, center=center)
    perm = torch.arange(64, dtype=torch.int32, device="cuda")
    sign = torch.ones(64, dtype=torch.int8, device="cuda")
    with pytest.raises(kq.KQError):
        kq.transform_quantize(X, kq.Xform.rpbh(perm, sign).with_pts(e))


def test_edge_rows(kq):
    """Zero rows, constant rows (centred: all zero), a single row, tiny and huge values."""
    K = 256
    rng = np.random.default_rng(5)
    X = rng.standard_normal((9, K)).astype(np.float16)
    X[0] = 0
    X[1] = np.float16(3.25)                 # constant token
    X[2] = np.float16(-0.0)
    X[3, :] = np.float16(6e-8)               # fp16 subnormals
    X[4] *= np.float16(1000)
    X[5, ::2] = 0
    perm, sign = synth.rpbh_params(K, 1, 0)
    A, B = synth.kron_factors(1, 0)
    for xf in ({"kind": "rpbh", "perm": perm, "sign": sign}, {"kind": "kron", "A": A, "B": B}):
        for center in (False, True):
            rep = _mx_check(kq, X, xf, center, f"edge {xf['kind']} center={center}")
            assert rep["code_mismatch"] == 0
    codes, scales, _ = _run(kq, X[:1], {"kind": "kron", "A": A, "B": B}, "mxfp4", False)
    assert np.all(codes == 0) and np.all(scales == 0)
    codes, scales, mu = _run(kq, X[1:2], {"kind": "rpbh", "perm": perm, "sign": sign}, "mxfp4", True)
    assert float(mu[0]) == 3.25 and np.all(codes == 0) and np.all(scales == 0)


def _crafted_e2m1_rows():
    """fp16 rows whose values land exactly on the E2M1 decision points once divided by the
    block's shared scale 2^e (e = floor(log2 max|x|) - 2): every rounding midpoint 0.25,
    0.75, 1.25, 1.75, 2.5, 3.5, 5 with both signs, values in the saturation band (6, 8),
    negative values that round to zero (code 0x8 by the sign rule), signed zeros, blocks
    whose maximum is exactly 2^k and one fp16 step below 2^k, and an all-zero block; at
    shared exponents from the fp16 subnormal range to near its top."""
    rng = np.random.default_rng(41)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    sat = [6.5, 7.0, 7.5, 7.9921875]
    grid = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    blocks = []
    for e in (-14, -9, -1, 0, 3, 12) * 6:
        base = [4.0] + mids + [-m for m in mids] + sat[:2] + [-v for v in sat[2:]] + \
               [-0.125, -0.25, -0.0, 0.0, -0.2421875, 0.125] + [-g for g in grid]
        assert len(base) == 32
        for _ in range(3):
            blocks.append(np.ldexp(np.array(rng.permutation(base), dtype=np.float64), e))
        k = e + 2
        top = np.float16(np.ldexp(1.0, k))
        below = np.nextafter(top, np.float16(0))
        for mx in (float(top), float(below)):           # block maximum 2^k and one fp16 step below
            b = np.ldexp(np.array(rng.permutation(mids + [-m for m in mids] + grid + [-g for g in grid] +
                                                   [0.0, -0.0, 0.25, -0.25]), dtype=np.float64), e - 1)
            b[rng.integers(32)] = -mx if rng.integers(2) else mx
            blocks.append(b)
    blocks.append(np.zeros(32))
    blocks.append(np.array([-0.0] * 32))
    while len(blocks) % 8:
        blocks.append(np.ldexp(np.array(rng.permutation([4.0] + mids + [-m for m in mids] + [0.0] * 17)), 2))
    rows = np.concatenate(blocks).reshape(-1, 256)
    x16 = rows.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), rows)      # every value is an fp16 number
    return x16


def test_e2m1_conversion_at_its_decision_points(kq):
    """The hardware E2M1 conversion on the identity path (exact float32 inputs, so no tie
    is allowed): codes and E8M0 bytes bit-equal to the oracle's round-to-nearest-even,
    saturating, sign-preserving rule at every decision point."""
    X16 = _crafted_e2m1_rows()
    xf = {"kind": "none"}
    codes, scales, _ = _run(kq, X16, xf, "mxfp4", False)
    ref = pipeline.transform_quantize(X16, xf, "mxfp4")
    got = mxfp4.unpack_nibbles(codes)
    bad = np.argwhere(got != ref["codes_unpacked"])
    print("crafted E2M1 blocks:", X16.shape, "mismatches", len(bad),
          [(int(m), int(k), float(X16[m, k]), int(got[m, k]), int(ref["codes_unpacked"][m, k])) for m, k in bad[:8]])
    assert len(bad) == 0
    assert np.array_equal(scales, ref["scales"])
    # the contract's corner cases, read off directly
    nib = got.reshape(-1, 32)
    xs = X16.astype(np.float64).reshape(-1, 32)
    sb = scales.reshape(-1).astype(np.int64)
    for b in range(len(xs)):
        e = sb[b] - 127
        s = np.ldexp(xs[b], -int(e)) if sb[b] else xs[b] * 0
        for v, c in zip(s, nib[b]):
            if v == 0.0:
                assert c == 0                               # exact zeros of either sign: code 0
            elif -0.25 <= v < 0:
                assert c == 0x8                             # negative, rounds to zero
            elif abs(v) >= 6.0:
                assert c & 7 == 7                           # saturates at 6
        amax = float(np.max(np.abs(xs[b])))
        if amax > 0:
            assert sb[b] == 127 + int(np.floor(np.log2(amax))) - 2


def test_single_row_and_ragged_block_count(kq):
    """M*K/32 not a multiple of 16 blocks (streaming kernel's ragged last chunk)."""
    A, B = synth.kron_factors(2, 0)
    xf = {"kind": "kron", "A": A, "B": B}
    for rows, K in ((1, 32), (1, 96), (3, 160), (7, 1152)):
        X16 = synth.activations(rows, K, 2, 2.0)
        rep = _mx_check(kq, X16, xf, False, f"ragged M={rows} K={K}")
        assert rep["code_mismatch"] <= 1


def _lm4_check(kq, X16, xf, label):
    codes_p, s_gpu, _ = _run(kq, X16, xf, "lm4", False)
    y, tau, _ = gpu_util.oracle_activation_reference(X16, xf, False, fmt="lm4")
    codes = mxfp4.unpack_nibbles(codes_p)
    # relative error bound of the kernel's scale: the float32 sum of squares (per-thread
    # chains of <= 32 terms, a 6-level wave tree, <= 16 wave partials), plus the effect
    # of the transformed values' own error, the division and the square root
    ss = np.sum(y * y, axis=1)
    s_rel = (gamma := 60 * gpu_util.U) + np.max(np.sum(2 * np.abs(y) * tau, axis=1) / np.maximum(ss, 1e-300)) + 4 * gpu_util.U
    rep = ties.classify_lm4(codes, s_gpu, y, tau, s_rel)
    msg = f"{label}: mismatches {rep['code_mismatch']}/{rep['codes']} ties {rep['code_ties']} errors {rep['errors'][:5]}"
    print(msg)
    assert not rep["errors"], msg
    assert rep["code_mismatch"] / rep["codes"] <= 1e-4, msg
    return rep


@pytest.mark.parametrize("layer,rows", [(0, 190), (2, 75)])
def test_lm4_codes_match_oracle(kq, layer, rows):
    c = synth.CONFIGS[2]
    _, K, _ = c["layers"][layer]
    X16 = synth.activations(rows, K, 2, c["sigma_mu"])
    _lm4_check(kq, X16, synth.xform_for(2, layer, K), f"cfg2 layer{layer} M={rows} K={K}")


@pytest.mark.parametrize("K,rows", [(32, 3), (2048, 9), (2080, 7), (16384, 5)])
def test_lm4_row_group_widths(kq, K, rows):
    """RPBH + per-token Lloyd-Max on the row-group kernel: four rows per group up to
    K = 2048 and two above, one block per row, the widest row, odd row counts."""
    X16 = synth.activations(rows, K, 25, 2.0)
    perm, sign = synth.rpbh_params(K, 25, 0)
    _lm4_check(kq, X16, {"kind": "rpbh", "perm": perm, "sign": sign}, f"lm4 K={K} M={rows}")


def test_lm4_zero_row(kq):
    K = 2240
    X16 = synth.activations(4, K, 2, 2.0)
    X16[2] = 0
    codes, s, _ = _run(kq, X16, synth.xform_for(2, 0, K), "lm4", False)
    assert s[2] == 0 and np.all(codes[2] == 0)


@pytest.mark.parametrize("K,rows", [(6144, 9), (6176, 9), (16384, 5)])
def test_rpbh_centred_row_group_widths(kq, K, rows):
    """The row-group kernel stages four rows per group up to K = 6144 and two above: both
    sides of the switch and the widest row, centred, odd row counts."""
    X16 = synth.activations(rows, K, 24, 4.0)
    perm, sign = synth.rpbh_params(K, 24, 0)
    _mx_check(kq, X16, {"kind": "rpbh", "perm": perm, "sign": sign}, True, f"rpbh centred K={K} M={rows}")


@pytest.mark.parametrize("kind,pts,M,K", [("kron", True, 8192, 4608), ("dense", True, 8192, 4608),
                                           ("none", False, 8191, 4608), ("kron", False, 8193, 1152),
                                           ("kron_blocks", False, 8192, 1152), ("kron_blocks", True, 8193, 4608)])
def test_streaming_forms_full_size_sampled(kq, kind, pts, M, K):
    """The streaming transforms at the PixArt-like sizes, on a grid of one resident round:
    every wavefront takes several steps with the next step's chunks in flight (and, with
    power-of-two scaling on the planted outlier channels, the next step's exponents); the
    per-block kernel with segments of several row groups.  Ragged M; parity on sampled rows
    (rows are independent)."""
    X16 = synth.activations(M, K, 19, 2.0)
    xf = {"kind": kind}
    if kind == "kron":
        xf["A"], xf["B"] = synth.kron_factors(19, 0)
    elif kind == "dense":
        xf["P"] = synth.dense_block(19, 0)
    elif kind == "kron_blocks":
        xf["A"], xf["B"] = synth.kron_block_factors(19, 0, K // 32)
    if pts:
        xf["pts"] = synth.pts_exponents(K, synth.outlier_channels(M, K, 19, 2.0))
    codes, scales, _ = _run(kq, X16, xf, "mxfp4", False)
    rows = np.unique(np.concatenate([np.arange(0, M, 131), [M - 2, M - 1]]))
    y, tau, _ = gpu_util.oracle_activation_reference(X16[rows], xf, False)
    gpu_util.assert_mx_parity(codes[rows], scales[rows], y, tau,
                              label=f"{kind} pts={pts} M={M} K={K} sampled {len(rows)}")


@pytest.mark.parametrize("cfg,layer", [(3, 0), (3, 2), (4, 0)])
def test_full_size_sampled_rows(kq, cfg, layer):
    """Full workload size in the launch configuration of the bench; parity on sampled rows
    (rows are independent)."""
    c = synth.CONFIGS[cfg]
    _, K, _ = c["layers"][layer]
    X16 = synth.activations(c["M"], K, cfg, c["sigma_mu"], c["frames"])
    xf = synth.xform_for(cfg, layer, K)
    codes, scales, mu = _run(kq, X16, xf, "mxfp4", c["center"])
    rows = np.unique(np.concatenate([np.arange(0, c["M"], 97), [c["M"] - 1]]))
    Xs = X16[rows]
    if c["center"]:
        gpu_util.check_mu(Xs, mu[rows])
    y, tau, _ = gpu_util.oracle_activation_reference(Xs, xf, c["center"], mu_gpu=None if mu is None else mu[rows])
    gpu_util.assert_mx_parity(codes[rows], scales[rows], y, tau, label=f"cfg{cfg} full M={c['M']} sampled {len(rows)}")
