"""The C-ABI library: loads, exports every symbol include/kq.h declares, and rejects bad
arguments on the host before anything is launched (no GPU needed)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import w4a4_post_quantization_amd as kq
from oracle import lloyd_max

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kq.lib_path()):
        pytest.fail("libkq.so is not built (run python -m w4a4_post_quantization_amd.build)")
    return kq.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"kq_transform_quantize", "kq_w4a4_linear", "kq_fold_inverse_into_weights",
            "kq_w4a4_linear_workspace_bytes", "kq_w4a4_linear_t", "kq_fold_inverse_into_weights_nk",
            "kq_abi_version", "kq_status_str"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", kq.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kq_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def test_abi_version_and_status_strings(lib):
    assert kq.abi_version() == 8
    for s in range(0, 8):
        assert kq.status_str(s).startswith("KQ_")
    assert "UNKNOWN" in kq.status_str(99)


def test_library_codebook_matches_oracle(lib):
    """The library's own Lloyd-Max solver (C++) and the oracle's (SciPy) agree."""
    for n, ref in ((16, lloyd_max.LEVELS16), (4, lloyd_max.LEVELS4)):
        got = np.array(kq.lloyd_max_levels(n))
        assert np.max(np.abs(got - ref)) <= 1e-12
    with pytest.raises(kq.KQError):
        kq.lloyd_max_levels(8)


def _xf(kind=1, K=64):
    x = kq._XformC()
    x.kind, x.reserved, x.K = kind, 0, K
    for i in range(4):
        x.A[5 * i] = 1.0
    for i in range(8):
        x.B[9 * i] = 1.0
    return x


FAKE = ctypes.c_void_p(0x100000)       # 16-byte aligned, never dereferenced on error paths
FAKE_ODD = ctypes.c_void_p(0x100008)


def test_transform_quantize_validation(lib):
    f = lib.kq_transform_quantize
    xf = _xf()
    assert f(ctypes.byref(xf), 0, 0, None, 4, 64, FAKE, FAKE, None, None) == 1          # NULL X
    assert f(None, 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 1                      # NULL xform
    assert f(ctypes.byref(xf), 0, 1, FAKE, 4, 64, FAKE, FAKE, None, None) == 1          # centre without mu
    assert f(ctypes.byref(xf), 0, 0, FAKE, 0, 64, FAKE, FAKE, None, None) == 2          # M < 1
    assert f(ctypes.byref(xf), 0, 0, FAKE, 4, 48, FAKE, FAKE, None, None) == 2          # K % 32
    assert f(ctypes.byref(xf), 0, 0, FAKE, 4, 96, FAKE, FAKE, None, None) == 2          # descriptor K
    assert f(ctypes.byref(xf), 7, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 4          # bad fmt
    assert f(ctypes.byref(xf), 0, 0, FAKE_ODD, 4, 64, FAKE, FAKE, None, None) == 3      # alignment
    bad = _xf(kind=9)
    assert f(ctypes.byref(bad), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 4         # bad kind
    rp = _xf(kind=2)
    assert f(ctypes.byref(rp), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 1          # RPBH without perm
    nan = _xf()
    nan.A[0] = float("nan")
    assert f(ctypes.byref(nan), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 5         # non-finite factor
    big = _xf(kind=2, K=65536 + 32)
    big.perm, big.sign = 0x100000, 0x100000
    assert f(ctypes.byref(big), 0, 0, FAKE, 4, 65536 + 32, FAKE, FAKE, None, None) == 4  # row too long


def test_pts_validation(lib):
    """Power-of-two channel scaling: streaming path only (MXFP4, no centring, not RPBH),
    a 16-byte aligned exponent vector."""
    f, g = lib.kq_transform_quantize, lib.kq_fold_inverse_into_weights
    xf = _xf()
    xf.pts = 0x100008
    assert f(ctypes.byref(xf), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 3          # misaligned pts
    assert g(ctypes.byref(xf), 0, FAKE, 64, 8, FAKE, FAKE, None, None) == 3
    xf.pts = 0x100000
    assert f(ctypes.byref(xf), 0, 1, FAKE, 4, 64, FAKE, FAKE, FAKE, None) == 4          # with centring
    assert f(ctypes.byref(xf), 1, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 4          # with LM4
    rp = _xf(kind=2)
    rp.perm, rp.sign, rp.pts = 0x100000, 0x100000, 0x100000
    assert f(ctypes.byref(rp), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 4          # with RPBH
    assert g(ctypes.byref(rp), 0, FAKE, 64, 8, FAKE, FAKE, None, None) == 4


def test_kron_blocks_validation(lib):
    """Per-block factors: the factor table must be given and 16-byte aligned; MXFP4 without
    centring only; kinds past the last are refused."""
    f, g = lib.kq_transform_quantize, lib.kq_fold_inverse_into_weights
    xf = _xf(kind=4)
    assert f(ctypes.byref(xf), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 1          # NULL AB
    assert g(ctypes.byref(xf), 0, FAKE, 64, 8, FAKE, FAKE, None, None) == 1
    xf.AB = 0x100008
    assert f(ctypes.byref(xf), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 3          # misaligned
    xf.AB = 0x100000
    assert f(ctypes.byref(xf), 0, 1, FAKE, 4, 64, FAKE, FAKE, FAKE, None) == 4          # with centring
    assert f(ctypes.byref(xf), 1, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 4          # with LM4
    bad = _xf(kind=5)
    assert f(ctypes.byref(bad), 0, 0, FAKE, 4, 64, FAKE, FAKE, None, None) == 4


@pytest.mark.parametrize("which", ["kq_fold_inverse_into_weights", "kq_fold_inverse_into_weights_nk"])
def test_fold_validation(lib, which):
    """Both weight layouts: W [K][N] takes (K, N), Wt [N][K] takes (N, K)."""
    g = getattr(lib, which)

    def f(xf, fmt, W, N, K, *rest):
        return g(xf, fmt, W, K, N, *rest) if which == "kq_fold_inverse_into_weights" else g(xf, fmt, W, N, K, *rest)
    xf = _xf()
    assert f(ctypes.byref(xf), 0, None, 8, 64, FAKE, FAKE, None, None) == 1
    assert f(ctypes.byref(xf), 1, FAKE, 8, 64, FAKE, FAKE, None, None) == 4             # LM4 is not a weight format
    assert f(ctypes.byref(xf), 0, FAKE, 8, 48, FAKE, FAKE, None, None) == 2             # K % 32
    assert f(ctypes.byref(xf), 0, FAKE, 0, 64, FAKE, FAKE, None, None) == 2             # N < 1
    assert f(ctypes.byref(xf), 0, FAKE_ODD, 8, 64, FAKE, FAKE, None, None) == 3
    sing = _xf()
    for i in range(16):
        sing.A[i] = 0.0
    assert f(ctypes.byref(sing), 0, FAKE, 8, 64, FAKE, FAKE, None, None) == 5           # singular A
    rank1 = _xf()
    for i in range(8):
        for j in range(8):
            rank1.B[8 * i + j] = float(i + 1)                                           # rank-1 B
    assert f(ctypes.byref(rank1), 0, FAKE, 8, 64, FAKE, FAKE, None, None) == 5


_LIN = dict(fmt=0, xc=FAKE, xs=FAKE, M=16, K=256, wc=FAKE, wsc=FAKE, N=32, r=0, mu=None, wbar=None, Y=FAKE)


def _common_linear_checks(call):
    assert call(Y=None) == 1
    assert call(N=0) == 2
    assert call(r=24) == 2
    assert call(mu=FAKE) == 2                          # mu without wbar
    assert call(K=96) == 4                             # MXFP4 needs K % 128
    assert call(N=40) == 4                             # N % 16
    assert call(fmt=5) == 4
    assert call(xc=FAKE_ODD) == 3
    assert call(mu=FAKE, wbar=FAKE_ODD) == 3           # the column sums are 16-byte aligned


def test_linear_t_validation(lib):
    f = lib.kq_w4a4_linear_t

    def call(**kw):
        a = {**_LIN, "T": None, "L2": None, **kw}
        return f(a["fmt"], a["xc"], a["xs"], a["M"], a["K"], a["wc"], a["wsc"], a["N"], a["T"], a["L2"],
                 a["r"], a["mu"], a["wbar"], a["Y"], None)
    _common_linear_checks(call)
    assert call(r=32) == 1                             # low rank without T/L2
    assert call(fmt=2, r=32, T=FAKE, L2=FAKE) == 4     # W2A4 has no low-rank branch
    assert call(r=32, T=FAKE_ODD, L2=FAKE) == 3


def test_linear_validation(lib):
    """The linear that runs the down-projection itself: X, L1, L2 and a workspace of at
    least kq_w4a4_linear_workspace_bytes(M, r) bytes, 256-byte aligned."""
    f = lib.kq_w4a4_linear
    need = kq.w4a4_linear_workspace_bytes(16, 32)

    def call(**kw):
        a = {**_LIN, "X": None, "L1": None, "L2": None, "ws": None, "wn": 0, **kw}
        return f(a["fmt"], a["xc"], a["xs"], a["M"], a["K"], a["wc"], a["wsc"], a["N"], a["X"], a["L1"], a["L2"],
                 a["r"], a["mu"], a["wbar"], a["Y"], a["ws"], a["wn"], None)
    _common_linear_checks(call)
    lr = dict(r=32, X=FAKE, L1=FAKE, L2=FAKE, ws=FAKE, wn=need)
    assert call(**dict(lr, X=None)) == 1               # low rank without X
    assert call(**dict(lr, L2=None)) == 1
    assert call(**dict(lr, ws=None)) == 7              # no workspace
    assert call(**dict(lr, wn=need - 1)) == 7          # too small
    assert call(**dict(lr, ws=ctypes.c_void_p(0x100010))) == 3
    assert call(**dict(lr, L1=FAKE_ODD)) == 3
    assert call(**dict(lr, fmt=2)) == 4                # W2A4 has no low-rank branch


def test_noalloc_linear_validation(lib):
    """The allocation-free linear refuses, before anything is launched, a T that would not
    fit its fixed scratch (KQ_ERR_WORKSPACE), and checks the other arguments like the
    workspace form."""
    f = lib.kq_w4a4_linear_noalloc

    def call(**kw):
        a = {**_LIN, "X": None, "L1": None, "L2": None, **kw}
        return f(a["fmt"], a["xc"], a["xs"], a["M"], a["K"], a["wc"], a["wsc"], a["N"], a["X"], a["L1"], a["L2"],
                 a["r"], a["mu"], a["wbar"], a["Y"], None)
    _common_linear_checks(call)
    lr = dict(r=64, X=FAKE, L1=FAKE, L2=FAKE)
    assert call(**dict(lr, X=None)) == 1
    assert call(**dict(lr, L1=FAKE_ODD)) == 3
    assert call(**dict(lr, M=(32 << 20) // 128 + 1)) == 7        # T of M x 64 fp16 beyond 32 MiB


def test_linear_workspace_size(lib):
    """T (fp16, padded to 256 bytes) plus the split-K partial sums; 0 without a branch;
    every rank the linear takes, 48 included; 0 for an invalid one."""
    for M in (1, 300, 4608, 17550):
        assert kq.w4a4_linear_workspace_bytes(M, 0) == 0
        for r in (16, 32, 48, 64):
            n = kq.w4a4_linear_workspace_bytes(M, r)
            assert n >= M * r * 2 and n % 256 == 0 or n >= M * r * 2
        assert kq.w4a4_linear_workspace_bytes(M, 24) == 0
    assert kq.w4a4_linear_workspace_bytes(0, 32) == 0
    # at least what the split down-projection alone uses at any K
    for K in (128, 3072, 12288):
        assert kq.w4a4_linear_workspace_bytes(4608, 32) >= kq.lowrank_down_workspace_bytes(4608, K, 32) + 4608 * 32 * 2


def test_clock_probe_validation(lib):
    f = lib.kq_clock_probe
    assert f(100, None, None) == 1
    assert f(0, FAKE, None) == 4
    assert f(1000001, FAKE, None) == 4
    assert f(100, ctypes.c_void_p(0x100004), None) == 3


def test_mfma_probe_validation(lib):
    f = lib.kq_mfma_fp4_probe
    assert f(10, 4, None, FAKE, None) == 1
    assert f(10, 4, FAKE, None, None) == 1
    assert f(0, 4, FAKE, FAKE, None) == 4
    assert f(1000001, 4, FAKE, FAKE, None) == 4
    assert f(10, 0, FAKE, FAKE, None) == 4
    assert f(10, 65537, FAKE, FAKE, None) == 4
    assert f(10, 4, ctypes.c_void_p(0x100004), FAKE, None) == 3
    assert f(10, 4, FAKE, ctypes.c_void_p(0x100002), None) == 3


def test_lowrank_validation(lib):
    f = lib.kq_lowrank_down
    assert f(None, FAKE, 4, 64, 32, FAKE, None, 0, None) == 1
    assert f(FAKE, FAKE, 4, 48, 32, FAKE, None, 0, None) == 2
    assert f(FAKE, FAKE, 4, 64, 8, FAKE, None, 0, None) == 2
    assert f(FAKE, FAKE, 0, 64, 32, FAKE, None, 0, None) == 2
    assert f(FAKE, FAKE_ODD, 4, 64, 32, FAKE, None, 0, None) == 3
    assert f(FAKE, FAKE, 4, 64, 32, FAKE, None, 1024, None) == 1      # size without a workspace
    assert f(FAKE, FAKE, 4, 64, 32, FAKE, FAKE_ODD, 1024, None) == 3


def test_transform_quantize_lowrank_validation(lib):
    """The fused pass: both calls' argument rules; the streaming kinds without centring and
    RPBH with or without it; no per-block factors, no power-of-two scaling."""
    f = lib.kq_transform_quantize_lowrank
    xf = _xf()
    args = lambda **kw: [kw.get("center", 0), kw.get("X", FAKE), kw.get("M", 4), kw.get("K", 64),
                         kw.get("codes", FAKE), FAKE, kw.get("mu", None), kw.get("L1", FAKE), kw.get("r", 32), FAKE,
                         kw.get("ws", None), kw.get("wn", 0), None]
    assert f(ctypes.byref(xf), *args(X=None)) == 1
    assert f(ctypes.byref(xf), *args(L1=None)) == 1
    assert f(None, *args()) == 1
    assert f(ctypes.byref(xf), *args(K=48)) == 2
    assert f(ctypes.byref(xf), *args(r=8)) == 2
    assert f(ctypes.byref(xf), *args(M=0)) == 2
    assert f(ctypes.byref(xf), *args(codes=FAKE_ODD)) == 3
    assert f(ctypes.byref(xf), *args(wn=1024)) == 1
    assert f(ctypes.byref(xf), *args(ws=FAKE_ODD, wn=1024)) == 3
    assert f(ctypes.byref(xf), *args(center=1, mu=FAKE)) == 4          # centring: RPBH only
    rp = _xf(kind=2)
    assert f(ctypes.byref(rp), *args()) == 1                            # RPBH without perm / sign
    rp.perm, rp.sign = 0x100000, 0x100000
    assert f(ctypes.byref(rp), *args(center=1)) == 1                    # centring without mu
    assert f(ctypes.byref(rp), *args(center=1, mu=ctypes.c_void_p(0x100001))) == 3
    kb = _xf(kind=4)
    kb.AB = 0x100000
    assert f(ctypes.byref(kb), *args()) == 4
    ps = _xf()
    ps.pts = 0x100000
    assert f(ctypes.byref(ps), *args()) == 4


def test_svd_lowrank_validation(lib):
    """Offline extraction: pointers, ranks, the oversampled width l, power steps, and a
    workspace of at least the reported size, 256-byte aligned."""
    f, wb = lib.kq_svd_lowrank, lib.kq_svd_lowrank_workspace_bytes
    need = wb(64, 96, 16, 24)
    assert need > 0 and wb(64, 96, 16, 16) == 0 and wb(64, 96, 8, 24) == 0
    big = need + 1024
    args = lambda **kw: [kw.get("W", FAKE), 64, kw.get("K", 96), kw.get("r", 16), FAKE, kw.get("l", 24),
                         kw.get("it", 4), FAKE, FAKE, FAKE, None, kw.get("ws", FAKE), kw.get("wn", big), None]
    assert f(*args(W=None)) == 1
    assert f(*args(ws=None)) == 1
    assert f(*args(r=8)) == 2
    assert f(*args(l=16)) == 2
    assert f(*args(l=97)) == 2
    assert f(*args(l=100, K=128)) == 2
    assert f(*args(it=17)) == 2
    assert f(*args(K=80)) == 2
    assert f(*args(wn=need - 1)) == 2
    assert f(*args(ws=ctypes.c_void_p(0x100010))) == 3


def test_lowrank_workspace_size(lib):
    """The split only pays for small M; the size is slices x M x r x 4 bytes, 0 when unsplit."""
    n = kq.lowrank_down_workspace_bytes(4608, 3072, 32)
    assert n > 0 and n % (4608 * 32 * 4) == 0
    assert kq.lowrank_down_workspace_bytes(4608, 128, 32) == 0          # one chunk of K: nothing to split
    assert kq.lowrank_down_workspace_bytes(4608, 3072, 8) == 0          # invalid rank
    assert kq.lowrank_down_workspace_bytes(4608, 3072, 48) % (4608 * 48 * 4) == 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    X = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        kq.transform_quantize(X, kq.Xform.none(64))
