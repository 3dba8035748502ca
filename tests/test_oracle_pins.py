"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test pins one part of the oracle to something other than the oracle itself:
values fixed by the format definition or a published table (tests/golden/),
brute force over small cases, closed forms, invariants and library routines.
All CPU, all fast.
"""

import fractions
import itertools
import math
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import linear, lloyd_max, mxfp4, pipeline, svd, ties, transforms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- P1: E2M1 RNE

def test_e2m1_golden_table():
    for v, c in _golden_rows("e2m1_rne.txt"):
        assert int(mxfp4.e2m1_encode(np.array(float(v)))) == int(c), v


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    vals = mxfp4.e2m1_decode(codes)
    back = mxfp4.e2m1_encode(vals)
    # -0 (code 8) decodes to 0.0 == -0.0, and an exact zero encodes as +0 (code 0)
    expect = codes.copy()
    expect[8] = 0
    assert np.array_equal(back, expect)
    assert sorted(set(np.abs(vals).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_brute_force_nearest_even():
    """Brute force: for many values, the chosen code is a nearest representable value,
    and on an exact midpoint it is the one with an even mantissa bit."""
    grid = mxfp4.e2m1_decode(np.arange(16, dtype=np.uint8))
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(-7, 7, 20000),
                           [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0]])
    got = mxfp4.e2m1_decode(mxfp4.e2m1_encode(vals))
    for v, g in zip(vals, got):
        dist = np.abs(grid - v)
        assert abs(g - v) == dist.min(), v
        near = np.unique(np.abs(grid[dist == dist.min()]))
        if len(near) == 2:      # a true tie: even code index, i.e. mantissa bit 0
            idx = int(np.where(mxfp4.E2M1_MAGNITUDES == abs(g))[0][0])
            assert idx % 2 == 0


def test_e2m1_boundaries_nextafter_and_saturation():
    bounds = [(0.25, 0, 1), (0.75, 1, 2), (1.25, 2, 3), (1.75, 3, 4), (2.5, 4, 5), (3.5, 5, 6), (5.0, 6, 7)]
    for b, below, above in bounds:
        assert int(mxfp4.e2m1_encode(np.nextafter(b, 0.0))) == below
        assert int(mxfp4.e2m1_encode(np.nextafter(b, 10.0))) == above
        assert int(mxfp4.e2m1_encode(-np.nextafter(b, 10.0))) == 8 + above
    for big in (6.0 * (1 + 2.0 ** -23), 7.99, 1e30):
        assert int(mxfp4.e2m1_encode(np.array(big))) == 7
        assert int(mxfp4.e2m1_encode(np.array(-big))) == 15
    assert int(mxfp4.e2m1_encode(np.array(-0.0))) == 0          # exact zero is +0
    assert int(mxfp4.e2m1_encode(np.array(-1e-300))) == 8       # negative rounding to zero


# ---------------------------------------------------------------- P2: E8M0

def test_e8m0_powers_of_two():
    for k in range(-120, 125):
        a = math.ldexp(1.0, k)
        e = int(mxfp4.e8m0_exponent(np.array([a]))[0])
        assert e == k - 2
        assert a * 2.0 ** -e == 4.0
        below = np.nextafter(a, 0.0)
        assert int(mxfp4.e8m0_exponent(np.array([below]))[0]) == k - 3
        # block maximum scaled into [4, 8)
        assert 4.0 <= below * 2.0 ** (-(k - 3)) < 8.0


def test_e8m0_clamps_and_zero():
    assert int(mxfp4.e8m0_exponent(np.array([0.0]))[0]) == -127
    assert int(mxfp4.e8m0_exponent(np.array([2.0 ** -140]))[0]) == -127
    assert int(mxfp4.e8m0_exponent(np.array([2.0 ** 140]))[0]) == 127
    codes, sb, e = mxfp4.quantize_blocks(np.zeros((1, 32)))
    assert sb[0, 0] == 0 and np.all(codes == 0)


def test_pack_nibble_order():
    codes = np.array([[1, 2, 15, 0]], dtype=np.uint8)
    p = mxfp4.pack_nibbles(codes)
    assert p.tolist() == [[0x21, 0x0F]]
    assert np.array_equal(mxfp4.unpack_nibbles(p), codes)


def test_quantization_error_bound():
    """P10: unsaturated values are within half a local grid step of their dequantized
    value; saturated values (above 6 after scaling) within 2 scale units."""
    rng = np.random.default_rng(1)
    y = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    codes, sb, e = mxfp4.quantize_blocks(y)
    d = mxfp4.dequantize(codes, sb)
    s = (y.reshape(64, 8, 32) * np.ldexp(1.0, -e)[..., None]).reshape(64, 256)
    err = np.abs(y - d) * np.repeat(np.ldexp(1.0, -e), 32, axis=1)
    a = np.abs(s)
    half_step = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    sat = a > 6
    assert np.all(err[~sat] <= half_step[~sat] + 1e-15)
    assert np.all(err[sat] < 2.0)
    assert np.all(a < 8.0) and np.all(a.reshape(64, 8, 32).max(axis=2) >= 4.0)


# ---------------------------------------------------------------- P3: Kronecker

def _random_factors(seed):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((4, 4)) + 2 * np.eye(4)).astype(np.float32)
    B = (rng.standard_normal((8, 8)) + 2 * np.eye(8)).astype(np.float32)
    return A, B


def test_kron_dense_matches_factored_form():
    """y = x (A (x) B) equals the mixed-product form Ym = A^T Xm B with Xm[i][j] = x[8i+j]."""
    A, B = _random_factors(2)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 32 * 6))
    y = transforms.apply_block_matrix(x, transforms.kron_block_matrix(A, B))
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    for m in range(16):
        for b in range(6):
            Xm = x[m, 32 * b:32 * b + 32].reshape(4, 8)
            Ym = A64.T @ Xm @ B64
            ref = Ym.reshape(32)
            got = y[m, 32 * b:32 * b + 32]
            assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_kron_entries_and_inverse():
    A, B = _random_factors(4)
    P = transforms.kron_block_matrix(A, B)
    for i, j, k, l in itertools.product(range(4), range(8), range(4), range(8)):
        assert P[8 * i + j, 8 * k + l] == np.float64(A[i, k]) * np.float64(B[j, l])
    Pinv = np.linalg.inv(P)
    ref = np.kron(np.linalg.inv(A.astype(np.float64)), np.linalg.inv(B.astype(np.float64)))
    assert np.max(np.abs(Pinv - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------------- P4: Hadamard / RPBH

def test_hadamard_sylvester_and_orthogonality():
    H = transforms.hadamard32()
    Hi = H.astype(np.int64)
    assert np.array_equal(Hi @ Hi.T, 32 * np.eye(32, dtype=np.int64))
    # Sylvester recursion built here, and the closed form (-1)^popcount(i & j)
    S = np.array([[1]], dtype=np.int64)
    for _ in range(5):
        S = np.block([[S, S], [S, -S]])
    assert np.array_equal(Hi, S)
    for i in range(32):
        for j in range(32):
            assert Hi[i, j] == (-1) ** bin(i & j).count("1")


def test_rpbh_orthogonal_and_matches_dense():
    K = 128
    rng = np.random.default_rng(5)
    perm = rng.permutation(K)
    sign = rng.choice([-1, 1], K)
    R = transforms.rpbh_dense(perm, sign)
    assert np.max(np.abs(R @ R.T - np.eye(K))) <= 1e-14
    x = rng.standard_normal((7, K))
    y = transforms.rpbh_apply(x, perm, sign)
    assert np.max(np.abs(y - x @ R)) <= 1e-13
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # the gather convention: (x Pi)_j = x_{pi(j)}
    xp = x @ R @ R.T
    assert np.allclose(xp, x, atol=1e-13)
    u = np.zeros(K)
    u[perm[3]] = 1.0
    v = transforms.rpbh_apply(u[None, :], perm, sign)[0]
    blk = 0
    assert np.allclose(np.abs(v[blk * 32:(blk + 1) * 32]), 1 / math.sqrt(32))


# ---------------------------------------------------------------- P5: the identity

@pytest.mark.parametrize("kind", ["kron", "rpbh", "dense", "kron_blocks"])
def test_invertible_transform_identity(kind):
    """(XP)(P^-1 W) = XW (KroQuant section 01; OrbitQuant section 03 W' = R^-1 W)."""
    rng = np.random.default_rng(6)
    K, N, M = 256, 96, 20
    X = rng.standard_normal((M, K))
    Wt = rng.standard_normal((N, K))             # W^T, [out][in]
    if kind == "kron":
        A, B = _random_factors(7)
        xf = {"kind": "kron", "A": A, "B": B}
    elif kind == "dense":
        xf = {"kind": "dense", "P": rng.standard_normal((32, 32)) + 4 * np.eye(32)}
    elif kind == "kron_blocks":
        import synth
        A, B = synth.kron_block_factors(7, 0, K // 32)
        xf = {"kind": "kron_blocks", "A": A, "B": B}
    else:
        xf = {"kind": "rpbh", "perm": rng.permutation(K), "sign": rng.choice([-1, 1], K)}
    lhs = pipeline.apply_transform(X, xf) @ pipeline.inverse_fold(Wt, xf).T
    rhs = X @ Wt.T
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(rhs)


def test_fold_solves_forward_transform():
    """P W' = W block by block (the fold is the inverse, checked with a linear solve)."""
    A, B = _random_factors(8)
    rng = np.random.default_rng(9)
    Wt = rng.standard_normal((10, 96))
    wpt = transforms.fold_kron(Wt, A, B)
    P = transforms.kron_block_matrix(A, B)
    for b in range(3):
        W_blk = Wt[:, 32 * b:32 * b + 32].T          # [32, N]
        sol = scipy.linalg.solve(P, W_blk)           # P^-1 W
        assert np.allclose(wpt[:, 32 * b:32 * b + 32].T, sol, rtol=1e-12, atol=1e-12)


def test_dense_block_special_cases():
    """The dense block transform (KroQuant section 01's P) against matrices whose action is
    known elementwise: the identity leaves x unchanged; a permutation matrix with
    P[pi(j), j] = 1 gathers y_j = x_{pi(j)} inside each block (the row-vector convention:
    a transposed P would scatter instead); a diagonal P scales; the fold with a diagonal P
    divides the weight rows by the same factors."""
    rng = np.random.default_rng(21)
    X = rng.standard_normal((5, 96))
    assert np.array_equal(pipeline.apply_transform(X, {"kind": "dense", "P": np.eye(32)}), X)
    pi = rng.permutation(32)
    P = np.zeros((32, 32))
    P[pi, np.arange(32)] = 1.0
    y = pipeline.apply_transform(X, {"kind": "dense", "P": P})
    for b in range(3):
        assert np.array_equal(y[:, 32 * b:32 * b + 32], X[:, 32 * b + pi])
    d = rng.uniform(0.5, 2.0, 32)
    y = pipeline.apply_transform(X, {"kind": "dense", "P": np.diag(d)})
    assert np.allclose(y, X * np.tile(d, 3)[None, :], rtol=0, atol=0)
    Wt = rng.standard_normal((7, 96))
    wpt = pipeline.inverse_fold(Wt, {"kind": "dense", "P": np.diag(d)})
    assert np.allclose(wpt, Wt / np.tile(d, 3)[None, :], rtol=1e-15)


def test_kron_blocks_reduce_to_shared_and_index_blocks():
    """Per-block factors: with every block given the same (A, B) they reduce to the shared
    Kronecker transform (pinned above against the factored form); with identity factors
    everywhere except block b, where A = diag(a) and B is the permutation matrix with
    B[pi(l), l] = 1, only block b changes and y[32b + 8k + l] = a_k x[32b + 8k + pi(l)]
    (np.kron order, row-vector convention, block b of the table acting on block b of x)."""
    rng = np.random.default_rng(23)
    K = 128
    X = rng.standard_normal((6, K))
    A, B = _random_factors(24)
    same = {"kind": "kron_blocks", "A": np.stack([A] * 4), "B": np.stack([B] * 4)}
    assert np.allclose(pipeline.apply_transform(X, same), pipeline.apply_transform(X, {"kind": "kron", "A": A, "B": B}),
                       rtol=1e-13, atol=1e-13)
    Ab = np.stack([np.eye(4)] * 4)
    Bb = np.stack([np.eye(8)] * 4)
    a, pi, b = rng.uniform(0.5, 2.0, 4), rng.permutation(8), 2
    Ab[b] = np.diag(a)
    Bb[b] = 0.0
    Bb[b][pi, np.arange(8)] = 1.0
    y = pipeline.apply_transform(X, {"kind": "kron_blocks", "A": Ab, "B": Bb})
    want = X.copy()
    for k in range(4):
        for l in range(8):
            want[:, 32 * b + 8 * k + l] = a[k] * X[:, 32 * b + 8 * k + pi[l]]
    assert np.array_equal(y, want)


def test_dense_orthogonal_preserves_block_norms():
    """An orthogonal dense P (the synthetic recipe's Haar factor) keeps every block's norm."""
    import synth
    P = synth.dense_block(3, 0).astype(np.float64)
    Q = P / np.linalg.norm(P, axis=0)[None, :]       # undo the column scales: Haar-orthogonal
    assert np.allclose(Q.T @ Q, np.eye(32), atol=1e-6)
    X = np.random.default_rng(22).standard_normal((4, 64))
    y = pipeline.apply_transform(X, {"kind": "dense", "P": Q})
    for b in range(2):
        assert np.allclose(np.linalg.norm(y[:, 32 * b:32 * b + 32], axis=1),
                           np.linalg.norm(X[:, 32 * b:32 * b + 32], axis=1), rtol=1e-6)


# ---------------------------------------------------------------- power-of-two channel scaling

def test_pts_fp16_shift_values():
    """DMQ's power-of-two scaling of fp16 activations against IEEE binary16 facts: in the
    normal range a power-of-two divide only lowers the exponent (exact); 2^-14 / 2 is the
    subnormal 2^-15; below the normal range the spacing is 2^-24, so 3 * 2^-24 / 2 = 1.5
    ulp rounds to the even 2 * 2^-24, 5 * 2^-24 / 2 = 2.5 ulp to 2 * 2^-24 and 7 * 2^-24 / 4
    = 1.75 ulp to 2 * 2^-24; 2^-24 / 4 rounds to zero; signs are kept."""
    x = np.array([[48.0, -2.0 ** -14, 3 * 2.0 ** -24, 5 * 2.0 ** -24, 7 * 2.0 ** -24, -(2.0 ** -24), 65504.0, 1.0]])
    e = np.array([5, 1, 1, 1, 2, 2, 15, 0])
    want = np.array([[1.5, -(2.0 ** -15), 2 * 2.0 ** -24, 2 * 2.0 ** -24, 2 * 2.0 ** -24, -0.0, 65504.0 / 32768, 1.0]])
    got = pipeline.apply_pts(x, e)
    assert np.array_equal(got, want)
    assert np.signbit(got[0, 5])


def test_pts_constant_shift_moves_only_the_mx_scale():
    """With the same exponent c on every channel, MXFP4 (a power-of-two shared scale per
    block) must give the same codes and every scale byte lowered by c, as long as the
    scaled values stay normal: a check that the scaling divides (not multiplies) and is a
    power of two."""
    rng = np.random.default_rng(30)
    X = (rng.standard_normal((6, 128)) * 8).astype(np.float16)
    X[np.abs(X.astype(np.float64)) < 2.0 ** -6] = np.float16(0.25)
    for c in (1, 3, 7):
        ref = pipeline.transform_quantize(X, {"kind": "none"})
        got = pipeline.transform_quantize(X, {"kind": "none", "pts": np.full(128, c)})
        assert np.array_equal(got["codes"], ref["codes"])
        assert np.array_equal(got["scales"].astype(int), ref["scales"].astype(int) - c)


@pytest.mark.parametrize("kind", ["none", "kron", "dense"])
def test_pts_fold_restores_the_product(kind):
    """(X D^-1 P)(P^-1 D W) = X W for activations whose scaled values stay fp16-normal
    (exact shift): checks the direction of the shift on both sides and that both index the
    input channel k (scaling the output channel instead breaks the product)."""
    import synth
    rng = np.random.default_rng(31)
    K, N = 96, 40
    X = (rng.standard_normal((5, K)) * 4).astype(np.float16)
    X[np.abs(X.astype(np.float64)) < 2.0 ** -4] = np.float16(0.5)
    Wt = rng.standard_normal((N, K))
    xf = {"kind": kind}
    if kind == "kron":
        A, B = synth.kron_factors(0, 0)
        xf.update(A=A, B=B)
    if kind == "dense":
        xf["P"] = synth.dense_block(0, 0)
    xf["pts"] = rng.integers(0, 9, size=K)
    y = pipeline.apply_transform(pipeline.apply_pts(X, xf["pts"]), xf)
    wt = pipeline.inverse_fold(Wt, xf)
    assert np.allclose(y @ wt.T, X.astype(np.float64) @ Wt.T, rtol=1e-9, atol=1e-9)
    wrong = dict(xf, pts=xf["pts"][::-1].copy())
    assert not np.allclose(y @ pipeline.inverse_fold(Wt, wrong).T, X.astype(np.float64) @ Wt.T, rtol=1e-3)


def test_pts_zero_exponents_change_nothing():
    rng = np.random.default_rng(32)
    X = (rng.standard_normal((4, 64)) * 3).astype(np.float16)
    a = pipeline.transform_quantize(X, {"kind": "none"})
    b = pipeline.transform_quantize(X, {"kind": "none", "pts": np.zeros(64, dtype=np.int8)})
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    with pytest.raises(ValueError):
        pipeline.transform_quantize(X, {"kind": "none", "pts": np.zeros(64)}, center=True)


# ---------------------------------------------------------------- low-rank extraction

def _haar_np(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))[None, :]


def test_svd_lowrank_recovers_a_known_spectrum():
    """Wt = U diag(s) V^T built from orthonormal U, V and distinct s: the rank-r part is
    U_r diag(s_r) V_r^T, the singular values are s, the residual's squared norm is the
    sum of the dropped s_i^2 (Eckart-Young), and the split is even:
    L2^T L2 = L1 L1^T = diag(s_r)."""
    rng = np.random.default_rng(40)
    N, K, r = 48, 80, 6
    U, V = _haar_np(rng, N, N), _haar_np(rng, K, N)
    s_true = np.sort(rng.uniform(0.1, 10.0, N))[::-1]
    Wt = (U * s_true[None, :]) @ V.T
    L1, L2, s = svd.svd_lowrank_f64(Wt, r)
    assert np.allclose(s, s_true, rtol=1e-12, atol=1e-12)
    best = (U[:, :r] * s_true[None, :r]) @ V[:, :r].T
    assert np.linalg.norm(L2 @ L1 - best) <= 1e-11 * np.linalg.norm(best)
    resid = np.linalg.norm(Wt - L2 @ L1) ** 2
    assert abs(resid - np.sum(s_true[r:] ** 2)) <= 1e-10 * np.sum(s_true ** 2)
    assert np.allclose(L2.T @ L2, np.diag(s_true[:r]), atol=1e-11)
    assert np.allclose(L1 @ L1.T, np.diag(s_true[:r]), atol=1e-11)


def test_svd_rank_one_matches_power_iteration():
    """Rank 1 of a small matrix against the textbook power iteration on Wt^T Wt, written
    here: the leading right singular vector and value agree."""
    rng = np.random.default_rng(41)
    Wt = rng.standard_normal((5, 7))
    v = np.ones(7)
    for _ in range(2000):
        v = Wt.T @ (Wt @ v)
        v /= np.linalg.norm(v)
    sigma = np.linalg.norm(Wt @ v)
    L1, L2, s = svd.svd_lowrank_f64(Wt, 1)
    assert abs(s[0] - sigma) <= 1e-12 * sigma
    assert np.allclose(L2 @ L1, np.outer(Wt @ v, v), atol=1e-10)


def test_svd_residual_uses_the_fp16_factors():
    """R is formed with the fp16 factors the branch will use: R64 + L2_16 L1_16 = Wt
    (float64, exact up to the final subtraction's rounding) and R is R64 rounded to fp16."""
    import synth
    Wt = synth.planted_lowrank_weights(96, 64, 3, 0, 8)
    out = svd.svd_lowrank(Wt, 8)
    back = out["R64"] + out["L2"].astype(np.float64) @ out["L1"].astype(np.float64)
    assert np.allclose(back, Wt.astype(np.float64), rtol=0, atol=1e-12)
    assert np.array_equal(out["R"], out["R64"].astype(np.float16))
    # the planted directions dominate: the residual is the bulk, far below W
    assert np.linalg.norm(out["R64"]) < 0.2 * np.linalg.norm(Wt.astype(np.float64))


# ---------------------------------------------------------------- P6: centring + rank-1

def test_centring_restore_exact():
    rng = np.random.default_rng(10)
    X = (rng.standard_normal((8, 64)) * 3 + 5).astype(np.float16)
    mu = pipeline.token_mean_f16(X)
    xc = pipeline.centre(X, mu)
    assert np.array_equal(xc + mu.astype(np.float64)[:, None], X.astype(np.float64))
    # exact rational arithmetic: (x - mu 1^T) W + mu (1^T W) = x W
    W = rng.integers(-5, 6, size=(64, 3))
    for m in range(2):
        xf = [fractions.Fraction(float(v)) for v in X[m]]
        muf = fractions.Fraction(float(mu[m]))
        for n in range(3):
            lhs = sum((xf[k] - muf) * int(W[k, n]) for k in range(64)) + muf * sum(int(W[k, n]) for k in range(64))
            rhs = sum(xf[k] * int(W[k, n]) for k in range(64))
            assert lhs == rhs


def test_centred_rotation_plus_rank1_equals_xw():
    rng = np.random.default_rng(11)
    K, N = 128, 40
    X = (rng.standard_normal((12, K)) + rng.normal(0, 4, (12, 1))).astype(np.float16)
    Wt = rng.standard_normal((N, K))
    xf = {"kind": "rpbh", "perm": rng.permutation(K), "sign": rng.choice([-1, 1], K)}
    mu = pipeline.token_mean_f16(X)
    y = pipeline.apply_transform(pipeline.centre(X, mu), xf)
    wbar = Wt.sum(axis=1)
    lhs = y @ pipeline.inverse_fold(Wt, xf).T + mu.astype(np.float64)[:, None] * wbar[None, :]
    rhs = X.astype(np.float64) @ Wt.T
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(rhs)


# ---------------------------------------------------------------- P7: mean survives Hadamard

def test_constant_token_survives_rotation_as_one_direction():
    """CentriQ abstract: a per-token mean survives the Hadamard rotation as one dominant
    coordinate per block; after centring it is gone."""
    K = 256
    rng = np.random.default_rng(12)
    perm, sign = rng.permutation(K), rng.choice([-1, 1], K)
    c = 2.75
    x = np.full((1, K), c)
    y = transforms.rpbh_apply(x, perm, sign)[0].reshape(K // 32, 32)
    for blk in y:
        nz = np.flatnonzero(np.abs(blk) > 1e-12)
        assert len(nz) == 1 and nz[0] == 0
        assert abs(abs(blk[0]) - math.sqrt(32) * c) <= 1e-12
    mu = pipeline.token_mean_f16(x.astype(np.float16))
    yc = pipeline.apply_transform(pipeline.centre(x.astype(np.float16), mu), {"kind": "rpbh", "perm": perm, "sign": sign})
    assert np.all(yc == 0.0)
    out = pipeline.transform_quantize(x.astype(np.float16), {"kind": "rpbh", "perm": perm, "sign": sign},
                                      center=True)
    assert np.all(out["codes"] == 0) and np.all(out["scales"] == 0)


# ---------------------------------------------------------------- P8: Lloyd-Max

def test_lloyd_max_against_published_table():
    rows = _golden_rows("lloyd_max_normal.txt")
    for r in rows:
        if r[0] == "levels":
            n = int(r[1])
            ref = np.array([float(v) for v in r[2:]])
            got = lloyd_max.lloyd_max_levels(n)
            assert np.allclose(got, ref, atol=6e-4), (n, got)
        elif r[0] == "thresholds":
            got = lloyd_max.thresholds(lloyd_max.lloyd_max_levels(int(r[1])))
            assert np.allclose(got, [float(v) for v in r[2:]], atol=6e-4)
        elif r[0] == "mse":
            got = lloyd_max.mse(lloyd_max.lloyd_max_levels(int(r[1])))
            assert abs(got - float(r[2])) <= 2e-3 * float(r[2])


def test_lloyd_max_fixed_point_and_empirical_mse():
    for n in (4, 16):
        lv = lloyd_max.lloyd_max_levels(n)
        assert lloyd_max.fixed_point_residual(lv) <= 1e-12
        assert np.all(np.diff(lv) > 0)
    rng = np.random.default_rng(13)
    z = rng.standard_normal((64, 4096))
    codes, s = lloyd_max.lm4_token_quantize(z)
    zq = lloyd_max.lm4_dequantize(codes, s)
    emp = np.mean((zq - z) ** 2)
    assert abs(emp - lloyd_max.mse(lloyd_max.LEVELS16)) < 1.5e-3


def test_lm4_edges():
    thr = lloyd_max.thresholds(lloyd_max.LEVELS16)
    # a value exactly on a threshold goes to the smaller magnitude; sign-magnitude layout
    assert int(lloyd_max.sign_magnitude_encode(np.array(thr[2]), thr)) == 2
    assert int(lloyd_max.sign_magnitude_encode(np.array(-thr[2]), thr)) == 8 + 2
    assert int(lloyd_max.sign_magnitude_encode(np.array(np.nextafter(thr[2], 9)), thr)) == 3
    assert int(lloyd_max.sign_magnitude_encode(np.array(100.0), thr)) == 7
    codes, s = lloyd_max.lm4_token_quantize(np.zeros((2, 64)))
    assert np.all(codes == 0) and np.all(s == 0)
    # decode undoes encode for level values
    lv = lloyd_max.LEVELS16
    c = lloyd_max.sign_magnitude_encode(np.concatenate([lv, -lv]), thr)
    assert np.array_equal(lloyd_max.sign_magnitude_decode(c, lv), np.concatenate([lv, -lv]))


def test_w2_pack_and_groups():
    rng = np.random.default_rng(14)
    wt = rng.standard_normal((6, 128))
    codes, s = lloyd_max.w2_group_quantize(wt)
    assert codes.max() <= 3 and s.dtype == np.float16
    p = lloyd_max.pack_2bit(codes)
    assert np.array_equal(lloyd_max.unpack_2bit(p), codes)
    assert lloyd_max.pack_2bit(np.array([[1, 2, 3, 0]], dtype=np.uint8)).tolist() == [[1 | (2 << 2) | (3 << 4)]]
    d = lloyd_max.w2_dequantize(codes, s)
    # every dequantized weight is +-level * its group scale
    g = np.abs(d.reshape(6, 4, 32)) / s.astype(np.float64)[..., None]
    assert np.all(np.isclose(g, lloyd_max.LEVELS4[0]) | np.isclose(g, lloyd_max.LEVELS4[1]))


# ---------------------------------------------------------------- P9: GEMM

def test_gemm_triple_loop_and_block_form():
    rng = np.random.default_rng(15)
    M, N, K = 3, 5, 64
    y = rng.standard_normal((M, K)) * 3
    w = rng.standard_normal((N, K))
    xc, xs, _ = mxfp4.quantize_blocks(y)
    wc, ws, _ = mxfp4.quantize_blocks(w)
    xp, wp = mxfp4.pack_nibbles(xc), mxfp4.pack_nibbles(wc)
    Xf = rng.standard_normal((M, K)).astype(np.float16)
    L1 = rng.standard_normal((4, K)).astype(np.float16)
    L2 = rng.standard_normal((N, 4)).astype(np.float16)
    mu = rng.standard_normal(M).astype(np.float16)
    wbar = rng.standard_normal(N).astype(np.float16)
    Y = linear.w4a4_linear(xp, xs, wp, ws, Xf, L1, L2, mu, wbar)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for b in range(K // 32):             # per-block scaled sums of code products
                sub = 0.0
                for k in range(32 * b, 32 * b + 32):
                    sub += mxfp4.e2m1_decode(xc[m, k]) * mxfp4.e2m1_decode(wc[n, k])
                acc += sub * 2.0 ** (int(xs[m, b]) - 127 + int(ws[n, b]) - 127)
            t = sum(sum(float(Xf[m, k]) * float(L1[r, k]) for k in range(K)) * float(L2[n, r]) for r in range(4))
            acc += t + float(mu[m]) * float(wbar[n])
            assert abs(Y[m, n] - acc) <= 1e-12 * (1 + abs(acc))


def test_gemm_sampled_rows_cols_match_full():
    rng = np.random.default_rng(16)
    M, N, K = 9, 11, 96
    xc, xs, _ = mxfp4.quantize_blocks(rng.standard_normal((M, K)))
    wc, ws, _ = mxfp4.quantize_blocks(rng.standard_normal((N, K)))
    xp, wp = mxfp4.pack_nibbles(xc), mxfp4.pack_nibbles(wc)
    full = linear.w4a4_linear(xp, xs, wp, ws)
    rows, cols = np.array([0, 4, 8]), np.array([1, 10])
    part = linear.w4a4_linear(xp, xs, wp, ws, rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])


# ---------------------------------------------------------------- P11: tie bound

def test_float32_kron_within_gamma_bound():
    """A float32 evaluation of the factored Kronecker product (the same operation count
    as a register implementation) stays within the gamma_n bound used to classify ties."""
    A, B = _random_factors(17)
    rng = np.random.default_rng(18)
    x16 = (rng.standard_normal((64, 32 * 8)) * np.where(rng.random(32 * 8) < 0.05, 50, 1)).astype(np.float16)
    x = x16.astype(np.float64)
    P = transforms.kron_block_matrix(A, B)
    y = transforms.apply_block_matrix(x, P)
    tau = ties.gamma_tau(12, transforms.apply_block_matrix(np.abs(x), np.abs(P)))
    A32, B32 = A.astype(np.float32), B.astype(np.float32)
    for m in range(64):
        for b in range(8):
            Xm = x16[m, 32 * b:32 * b + 32].astype(np.float32).reshape(4, 8)
            Z = np.zeros((4, 8), np.float32)
            for j in range(8):
                Z = (Z + Xm[:, j:j + 1] * B32[j:j + 1, :]).astype(np.float32)
            Y = np.zeros((4, 8), np.float32)
            for i in range(4):
                Y = (Y + A32[i:i + 1, :].T * Z[i:i + 1, :]).astype(np.float32)
            err = np.abs(Y.reshape(32).astype(np.float64) - y[m, 32 * b:32 * b + 32])
            assert np.all(err <= tau[m, 32 * b:32 * b + 32])


def test_tie_classifier_catches_planted_errors():
    """A code flipped far from any boundary is an error; a float32 rounding of a value on
    a boundary is a tie."""
    rng = np.random.default_rng(19)
    y = rng.standard_normal((4, 64)) * 3
    tau = np.full(y.shape, 1e-6)
    codes, sb, e = mxfp4.quantize_blocks(y)
    rep = ties.classify_mxfp4(codes, sb, y, tau)
    assert rep["errors"] == [] and rep["code_mismatch"] == 0
    bad = codes.copy()
    bad[1, 5] ^= 0x3            # flip magnitude bits: not a rounding neighbour
    rep = ties.classify_mxfp4(bad, sb, y, tau)
    assert len(rep["errors"]) == 1
    # a value exactly on a boundary, and a "kernel" that picked the other side of it
    y2 = np.zeros((1, 32))
    y2[0, 0], y2[0, 1], y2[0, 2] = 4.0, 1.25, -2.5          # block max 4 -> e = 0
    c2, s2, e2 = mxfp4.quantize_blocks(y2)
    assert int(e2[0, 0]) == 0 and c2[0, 1] == 2 and c2[0, 2] == 12
    alt = c2.copy()
    alt[0, 1] = 3              # 1.5 instead of the even 1.0
    alt[0, 2] = 13             # -3 instead of the even -2
    rep = ties.classify_mxfp4(alt, s2, y2, np.full(y2.shape, 1e-9))
    assert rep["errors"] == [] and rep["code_ties"] == 2
    rep = ties.classify_mxfp4(alt, s2, y2, np.zeros(y2.shape))   # no error budget: not a tie
    assert len(rep["errors"]) == 2
    bad_scale = sb.copy()
    bad_scale[0, 0] += 3
    rep = ties.classify_mxfp4(codes, bad_scale, y, tau)
    assert any(err[0] == "scale" for err in rep["errors"])


def test_lm4_tie_classifier_catches_planted_errors():
    """The Lloyd-Max classifier: exact codes pass; a code flipped on a value far from every
    threshold is an error; a scale outside its bound is an error; a value on a threshold
    with a "kernel" code on either side is a tie only when the error budget reaches it;
    and the budget is not wider than the bound it is given (a value a few budgets away
    from the threshold, flipped across it, is an error)."""
    rng = np.random.default_rng(31)
    y = rng.standard_normal((3, 256))
    codes, s = lloyd_max.lm4_token_quantize(y)
    thr = lloyd_max.thresholds(lloyd_max.LEVELS16)
    tau = np.full(y.shape, 1e-9)
    rel = 1e-7
    rep = ties.classify_lm4(codes, s, y, tau, rel)
    assert rep["errors"] == [] and rep["code_mismatch"] == 0 and rep["scale_errors"] == 0
    # a non-tie flip: the value with the largest distance to any threshold, moved one level
    v = y / s.astype(np.float64)[:, None]
    dist = np.min(np.abs(np.abs(v)[..., None] - thr), axis=-1)
    m, k = np.unravel_index(np.argmax(dist), v.shape)
    bad = codes.copy()
    bad[m, k] = (bad[m, k] & 8) | ((bad[m, k] & 7) ^ 1)
    rep = ties.classify_lm4(bad, s, y, tau, rel)
    assert len(rep["errors"]) == 1 and rep["errors"][0][0] == "code" and rep["code_ties"] == 0
    # a scale off by far more than its bound
    s_bad = s.copy()
    s_bad[1] *= np.float32(1.001)
    rep = ties.classify_lm4(codes, s_bad, y, tau, rel)
    assert any(e[0] == "scale" and e[1] == 1 for e in rep["errors"])
    # a value exactly on a threshold: the oracle takes the smaller magnitude; a kernel that
    # took the larger one is a tie with an error budget, an error without one
    y2 = rng.standard_normal((1, 64))
    i = 5
    for _ in range(50):           # y_i moves s_t: iterate to the fixed point of the stored scale
        c2, s2v = lloyd_max.lm4_token_quantize(y2)
        on = float(thr[3]) * float(s2v[0])
        if y2[0, i] == on:
            break
        y2[0, i] = on
    c2, s2v = lloyd_max.lm4_token_quantize(y2)
    v_i = y2[0, i] / float(s2v[0])
    assert abs(v_i - thr[3]) <= 4e-16 * thr[3]
    alt = c2.copy()
    alt[0, i] = 4 if int(c2[0, i]) == 3 else 3
    rep = ties.classify_lm4(alt, s2v, y2, np.full(y2.shape, 1e-9), 1e-7)
    assert rep["errors"] == [] and rep["code_ties"] == 1
    rep = ties.classify_lm4(alt, s2v, y2, np.zeros(y2.shape), 0.0)
    if abs(v_i - thr[3]) > 0:                       # off the threshold by rounding: an error
        assert len(rep["errors"]) == 1
    # a value five budgets beyond the threshold, coded on the other side: an error
    t_abs = 1e-7
    y3 = y2.copy()
    d = float(s2v[0]) * (t_abs / float(s2v[0]) + abs(thr[3]) * (1e-7 + 2 * ties.U32))
    y3[0, i] = on + 5 * d
    c3, s3 = lloyd_max.lm4_token_quantize(y3)
    alt3 = c3.copy()
    alt3[0, i] = 3 if int(c3[0, i]) == 4 else 4
    rep = ties.classify_lm4(alt3, s3, y3, np.full(y3.shape, t_abs), 1e-7)
    assert len(rep["errors"]) == 1 and rep["code_ties"] == 0


@pytest.mark.parametrize("kind", ["rpbh", "kron"])
def test_fold_wbar_restores_the_mean(kind):
    """CentriQ abstract: with x centred by its stored fp16 mean, the fold's own outputs --
    W'^T and the fp16 column sums wbar -- give back x W:
        (x - mu 1^T) P . (P^-1 W) + mu wbar^T = x W
    up to the fp16 rounding of wbar, which bounds the residual by |mu| |wbar - 1^T W|.
    A wbar taken from the folded W' (a plausible slip) breaks the identity."""
    rng = np.random.default_rng(32)
    K, N, M = 256, 48, 10
    X = (rng.standard_normal((M, K)) + rng.normal(0, 4, (M, 1))).astype(np.float16)
    Wt = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float16)
    if kind == "rpbh":
        xf = {"kind": "rpbh", "perm": rng.permutation(K), "sign": rng.choice([-1, 1], K)}
    else:
        A = rng.standard_normal((4, 4)) + 2 * np.eye(4)
        B = rng.standard_normal((8, 8)) + 3 * np.eye(8)
        xf = {"kind": "kron", "A": A.astype(np.float32), "B": B.astype(np.float32)}
    fw = pipeline.fold_weights(Wt, xf, "mxfp4")
    a = pipeline.transform_quantize(X, xf, "mxfp4", center=True)
    mu = a["mu"].astype(np.float64)
    rhs = X.astype(np.float64) @ Wt.astype(np.float64).T
    lhs = a["y"] @ fw["wt"].T + mu[:, None] * fw["wbar"].astype(np.float64)[None, :]
    exact_wbar = Wt.astype(np.float64).sum(axis=1)
    bound = np.abs(mu)[:, None] * np.abs(fw["wbar"].astype(np.float64) - exact_wbar)[None, :]
    assert np.all(np.abs(lhs - rhs) <= bound + 1e-9 * np.max(np.abs(rhs)))
    # the same identity with exact wbar holds to fp64 rounding
    lhs64 = a["y"] @ fw["wt"].T + mu[:, None] * exact_wbar[None, :]
    assert np.linalg.norm(lhs64 - rhs) <= 1e-12 * np.linalg.norm(rhs)
    # wbar from the folded weights: fails by far more than the fp16 rounding
    wrong = fw["wt"].sum(axis=1).astype(np.float16).astype(np.float64)
    lhs_bad = a["y"] @ fw["wt"].T + mu[:, None] * wrong[None, :]
    assert np.max(np.abs(lhs_bad - rhs)) > 100 * (np.max(bound) + 1e-9 * np.max(np.abs(rhs)))


def test_mean_tie_rule():
    x = np.array([1.0, np.float16(1.0) + np.float16(2.0 ** -10)], dtype=np.float16)
    exact = float(np.mean(x.astype(np.float64)))     # the fp16 midpoint of 1 and 1+2^-10
    lo, hi = np.float16(1.0), np.float16(1.0 + 2.0 ** -10)
    assert exact == 0.5 * (float(lo) + float(hi))
    assert ties.mean_tie(x, lo, hi, 2)
    assert not ties.mean_tie(x, np.float16(2.0), hi, 2)
