"""Python binding of libkq (the MI355X HIP library for the online 4-bit activation path).

Argument marshalling only: every step of the path runs in the library's HIP kernels.
Tensors are torch tensors on the ROCm device (PyTorch provides device memory and the
stream); outputs are allocated here when not given.  The binding fails loudly if the
library is missing: there is no fallback.

    xf = kq.Xform.kron(A, B, K)                     # or Xform.rpbh(perm, sign), Xform.none(K)
    codes, scales, mu = kq.transform_quantize(X, xf, fmt="mxfp4", center=False)
    wcodes, wscales, wbar = kq.fold_inverse_into_weights(W, xf, fmt="mxfp4")     # W [K][N]
    Y = kq.w4a4_linear(codes, scales, wcodes, wscales, X=X, L1=L1, L2=L2, mu=mu, wbar=wbar)
    # or, with the down-projection done separately (or fused into the transform):
    T = kq.lowrank_down(X, L1)
    Y = kq.w4a4_linear_t(codes, scales, wcodes, wscales, T=T, L2=L2, mu=mu, wbar=wbar)

Outputs and workspaces that the binding allocates itself are marked as used on the stream
the call runs on (``record_stream``), so torch's allocator does not hand their memory to
another stream's work before the call has finished there.
"""

import ctypes
import os

__all__ = ["mfma_fp4_probe", "load", "lib_path", "abi_version", "status_str", "lloyd_max_levels", "Xform",
           "transform_quantize", "fold_inverse_into_weights", "fold_inverse_into_weights_nk",
           "w4a4_linear", "w4a4_linear_t", "w4a4_linear_workspace_bytes",
           "lowrank_down", "lowrank_down_workspace_bytes", "transform_quantize_lowrank",
           "svd_lowrank", "svd_lowrank_workspace_bytes", "KQError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

KQ_OK = 0
XFORM_NONE, XFORM_KRON, XFORM_RPBH, XFORM_DENSE, XFORM_KRON_BLOCKS = 0, 1, 2, 3, 4
FMT_MXFP4, FMT_LM4, FMT_LM2 = 0, 1, 2
_FMT = {"mxfp4": FMT_MXFP4, "lm4": FMT_LM4, "lm2": FMT_LM2}


class KQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {status_str(status)}")
        self.status = status


class _XformC(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_int32), ("K", ctypes.c_int64),
                ("A", ctypes.c_float * 16), ("B", ctypes.c_float * 64),
                ("perm", ctypes.c_void_p), ("sign", ctypes.c_void_p), ("P", ctypes.c_void_p),
                ("AB", ctypes.c_void_p), ("pts", ctypes.c_void_p)]


def lib_path():
    return os.path.join(_HERE, "libkq.so")


def load():
    """Load libkq.so (built in-tree by build.py); raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m w4a4_post_quantization_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kq_abi_version.restype = i32
    lib.kq_abi_version.argtypes = []
    lib.kq_status_str.restype = ctypes.c_char_p
    lib.kq_status_str.argtypes = [i32]
    lib.kq_clock_probe.restype = i32
    lib.kq_clock_probe.argtypes = [i32, vp, vp]
    lib.kq_mfma_fp4_probe.restype = i32
    lib.kq_mfma_fp4_probe.argtypes = [i32, i32, vp, vp, vp]
    lib.kq_lloyd_max_levels.restype = i32
    lib.kq_lloyd_max_levels.argtypes = [i32, ctypes.POINTER(ctypes.c_double)]
    lib.kq_transform_quantize.restype = i32
    lib.kq_transform_quantize.argtypes = [ctypes.POINTER(_XformC), i32, i32, vp, i64, i64, vp, vp, vp, vp]
    lib.kq_fold_inverse_into_weights.restype = i32
    lib.kq_fold_inverse_into_weights.argtypes = [ctypes.POINTER(_XformC), i32, vp, i64, i64, vp, vp, vp, vp]
    lib.kq_fold_inverse_into_weights_nk.restype = i32
    lib.kq_fold_inverse_into_weights_nk.argtypes = [ctypes.POINTER(_XformC), i32, vp, i64, i64, vp, vp, vp, vp]
    lib.kq_lowrank_down.restype = i32
    lib.kq_lowrank_down.argtypes = [vp, vp, i64, i64, i32, vp, vp, ctypes.c_size_t, vp]
    lib.kq_lowrank_down_workspace_bytes.restype = ctypes.c_size_t
    lib.kq_lowrank_down_workspace_bytes.argtypes = [i64, i64, i32]
    lib.kq_transform_quantize_lowrank.restype = i32
    lib.kq_transform_quantize_lowrank.argtypes = [ctypes.POINTER(_XformC), i32, vp, i64, i64, vp, vp, vp, vp, i32,
                                                  vp, vp, ctypes.c_size_t, vp]
    lib.kq_svd_lowrank_workspace_bytes.restype = ctypes.c_size_t
    lib.kq_svd_lowrank_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.kq_svd_lowrank.restype = i32
    lib.kq_svd_lowrank.argtypes = [vp, i64, i64, i32, vp, i32, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.kq_w4a4_linear_workspace_bytes.restype = ctypes.c_size_t
    lib.kq_w4a4_linear_workspace_bytes.argtypes = [i64, i32]
    lib.kq_w4a4_linear.restype = i32
    lib.kq_w4a4_linear.argtypes = [i32, vp, vp, i64, i64, vp, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.kq_w4a4_linear_noalloc.restype = i32
    lib.kq_w4a4_linear_noalloc.argtypes = [i32, vp, vp, i64, i64, vp, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.kq_w4a4_linear_t.restype = i32
    lib.kq_w4a4_linear_t.argtypes = [i32, vp, vp, i64, i64, vp, vp, i64, vp, vp, i32, vp, vp, vp, vp]
    _LIB = lib
    return lib


def abi_version():
    return int(load().kq_abi_version())


def status_str(s):
    return load().kq_status_str(int(s)).decode()


def clock_probe(spin_us, out=None, stream=None):
    """Launch the shader-clock probe on `stream` (see kq_clock_probe): returns the device
    uint64 [2] tensor that will hold (shader cycles, 100 MHz reference ticks)."""
    torch = _torch()
    if out is None:
        out = torch.empty((2,), dtype=torch.int64, device="cuda")      # no fill kernel to race with
        _on_stream(stream, out)
    _check(out, "out", torch.int64, (2,))
    s = load().kq_clock_probe(int(spin_us), _ptr(out), _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_clock_probe")
    return out


def mfma_fp4_probe(iters, workgroups, codes, out=None, stream=None):
    """Launch the FP4 matrix-core rate probe on `stream` (see kq_mfma_fp4_probe): `codes` is a
    device uint8 tensor of at least 2048 bytes (its first 2048 are the operands); returns the
    float32 [4 * workgroups] tensor of per-wavefront sums.  The caller times the launch; the
    work is 64 * iters * workgroups products of 2 * 32 * 32 * 64 flops."""
    torch = _torch()
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous() or codes.numel() < 2048:
        raise ValueError("codes must be a contiguous device uint8 tensor of at least 2048 bytes")
    if out is None:
        out = torch.empty((4 * int(workgroups),), dtype=torch.float32, device=codes.device)
        _on_stream(stream, out)
    _check(out, "out", torch.float32, (4 * int(workgroups),))
    s = load().kq_mfma_fp4_probe(int(iters), int(workgroups), _ptr(codes), _ptr(out), _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_mfma_fp4_probe")
    return out


def lloyd_max_levels(n):
    """Positive levels of the library's n-level (4 or 16) Lloyd-Max codebook (host call)."""
    out = (ctypes.c_double * (n // 2))()
    s = load().kq_lloyd_max_levels(n, out)
    if s != KQ_OK:
        raise KQError(s, "kq_lloyd_max_levels")
    return [float(v) for v in out]


# ------------------------------------------------------------------ marshalling helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream, *made):
    """Tensors this binding allocated on torch's current stream but handed to a call on
    another stream: record that stream on them, so their memory is not reused before the
    call has finished there (torch's caching allocator otherwise only waits for the
    stream they were allocated on)."""
    if stream is None:
        return
    torch = _torch()
    if stream == torch.cuda.current_stream():
        return
    for t in made:
        if t is not None:
            t.record_stream(stream)


def _check(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


class Xform:
    """One layer's block transform descriptor (KRON_4X8, RPBH_32, DENSE_32 or NONE)."""

    def __init__(self, kind, K, A=None, B=None, perm=None, sign=None, P=None, AB=None, pts=None):
        self.kind, self.K = kind, int(K)
        self._c = _XformC()
        self._c.kind, self._c.reserved, self._c.K = kind, 0, self.K
        if kind == XFORM_KRON:
            a = [float(v) for v in _flat(A)]
            b = [float(v) for v in _flat(B)]
            if len(a) != 16 or len(b) != 64:
                raise ValueError("A must be 4x4 and B 8x8")
            self._c.A[:] = a
            self._c.B[:] = b
        self.perm, self.sign = perm, sign      # keep the device arrays alive
        if kind == XFORM_RPBH:
            torch = _torch()
            _check(perm, "perm", torch.int32, (self.K,))
            _check(sign, "sign", torch.int8, (self.K,))
            self._c.perm, self._c.sign = perm.data_ptr(), sign.data_ptr()
        self.P = P
        if kind == XFORM_DENSE:
            torch = _torch()
            _check(P, "P", torch.float32, (32, 32))
            self._c.P = P.data_ptr()
        self.AB = AB
        if kind == XFORM_KRON_BLOCKS:
            _check(AB, "AB", _torch().float32, (self.K // 32, 80))
            self._c.AB = AB.data_ptr()
        self.pts = pts
        if pts is not None:
            _check(pts, "pts", _torch().int8, (self.K,))
            self._c.pts = pts.data_ptr()

    def with_pts(self, pts):
        """The same transform preceded by power-of-two channel scaling: pts is an int8 [K]
        device tensor of exponents (0..15); x_k -> fp16(x_k 2^-pts[k]), weights x 2^pts[k]."""
        return Xform(self.kind, self.K, A=list(self._c.A), B=list(self._c.B), perm=self.perm, sign=self.sign,
                     P=self.P, AB=self.AB, pts=pts)

    @classmethod
    def kron(cls, A, B, K):
        return cls(XFORM_KRON, K, A=A, B=B)

    @classmethod
    def kron_blocks(cls, AB, K):
        """AB: float32 [K/32][80] device tensor, row b = A_b (4x4) then B_b (8x8), row-major;
        block b of every token becomes x_b . (A_b (x) B_b)."""
        return cls(XFORM_KRON_BLOCKS, K, AB=AB)

    @staticmethod
    def pack_block_factors(A, B):
        """Host helper: A [nb][4][4], B [nb][8][8] -> the float32 [nb][80] table (numpy)."""
        import numpy as np
        A = np.asarray(A, dtype=np.float32)
        B = np.asarray(B, dtype=np.float32)
        return np.ascontiguousarray(np.concatenate([A.reshape(len(A), 16), B.reshape(len(B), 64)], axis=1))

    @classmethod
    def dense(cls, P, K):
        """P: float32 [32][32] device tensor, y_b = x_b . P for every block."""
        return cls(XFORM_DENSE, K, P=P)

    @classmethod
    def rpbh(cls, perm, sign):
        return cls(XFORM_RPBH, perm.shape[0], perm=perm, sign=sign)

    @classmethod
    def none(cls, K):
        return cls(XFORM_NONE, K)

    def c(self):
        return ctypes.byref(self._c)


def _flat(a):
    try:
        import numpy as np
        return np.asarray(a, dtype=np.float32).reshape(-1).tolist()
    except Exception:
        return list(a)


def transform_quantize(X, xform, fmt="mxfp4", center=False, codes=None, scales=None, mu=None, stream=None):
    """[centre] -> block transform -> 4-bit quantize + pack.  Returns (codes, scales, mu)."""
    torch = _torch()
    _check(X, "X", torch.float16)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M, K]")
    M, K = X.shape
    f = _FMT[fmt]
    if f not in (FMT_MXFP4, FMT_LM4):
        raise ValueError("fmt must be 'mxfp4' or 'lm4'")
    dev = X.device
    made = []
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        made.append(codes)
    _check(codes, "codes", torch.uint8, (M, K // 2))
    if scales is None:
        scales = torch.empty((M, K // 32) if f == FMT_MXFP4 else (M,),
                             dtype=torch.uint8 if f == FMT_MXFP4 else torch.float32, device=dev)
        made.append(scales)
    if f == FMT_MXFP4:
        _check(scales, "scales", torch.uint8, (M, K // 32))
    else:
        _check(scales, "scales", torch.float32, (M,))
    if center:
        if mu is None:
            mu = torch.empty((M,), dtype=torch.float16, device=dev)
            made.append(mu)
        _check(mu, "mu", torch.float16, (M,))
    else:
        mu = None
    _on_stream(stream, *made)
    s = load().kq_transform_quantize(xform.c(), f, int(bool(center)), _ptr(X), M, K, _ptr(codes), _ptr(scales),
                                     _ptr(mu), _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_transform_quantize")
    return codes, scales, mu


def _fold(name, W, N, K, xform, fmt, with_wbar, stream):
    torch = _torch()
    f = _FMT[fmt]
    dev = W.device
    if f == FMT_MXFP4:
        wcodes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        wscales = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    elif f == FMT_LM2:
        wcodes = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
        wscales = torch.empty((N, K // 32), dtype=torch.float16, device=dev)
    else:
        raise ValueError("fmt must be 'mxfp4' or 'lm2'")
    wbar = torch.empty((N,), dtype=torch.float16, device=dev) if with_wbar else None
    _on_stream(stream, wcodes, wscales, wbar)
    fn = getattr(load(), name)
    if name == "kq_fold_inverse_into_weights":
        s = fn(xform.c(), f, _ptr(W), K, N, _ptr(wcodes), _ptr(wscales), _ptr(wbar), _stream(stream))
    else:
        s = fn(xform.c(), f, _ptr(W), N, K, _ptr(wcodes), _ptr(wscales), _ptr(wbar), _stream(stream))
    if s != KQ_OK:
        raise KQError(s, name)
    return wcodes, wscales, wbar


def fold_inverse_into_weights(W, xform, fmt="mxfp4", with_wbar=True, stream=None):
    """Offline: W' = P^-1 W, quantized along K.  W is fp16 [K][N] (Y = X W).
    Returns (wcodes [N][K/2], wscales [N][K/32], wbar [N] or None)."""
    torch = _torch()
    _check(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [K, N]")
    K, N = W.shape
    return _fold("kq_fold_inverse_into_weights", W, N, K, xform, fmt, with_wbar, stream)


def fold_inverse_into_weights_nk(Wt, xform, fmt="mxfp4", with_wbar=True, stream=None):
    """The same fold for weights in the [out][in] layout: Wt is fp16 [N][K]."""
    torch = _torch()
    _check(Wt, "Wt", torch.float16)
    if Wt.dim() != 2:
        raise ValueError("Wt must be 2-D [N, K]")
    N, K = Wt.shape
    return _fold("kq_fold_inverse_into_weights_nk", Wt, N, K, xform, fmt, with_wbar, stream)


def lowrank_down_workspace_bytes(M, K, r):
    """Workspace bytes that let kq_lowrank_down split K over workgroups (0: no split)."""
    return int(load().kq_lowrank_down_workspace_bytes(M, K, r))


def lowrank_down(X, L1, T=None, workspace=None, stream=None):
    """T = fp16(X L1^T): the low-rank branch's down-projection (fp16 [M][r]).  workspace:
    a uint8 device tensor for the split-K partials; by default one of the size
    lowrank_down_workspace_bytes is taken from torch's allocator."""
    torch = _torch()
    _check(X, "X", torch.float16)
    M, K = X.shape
    r = L1.shape[0]
    _check(L1, "L1", torch.float16, (r, K))
    made = []
    if T is None:
        T = torch.empty((M, r), dtype=torch.float16, device=X.device)
        made.append(T)
    _check(T, "T", torch.float16, (M, r))
    if workspace is None:
        nb = lowrank_down_workspace_bytes(M, K, r)
        workspace = torch.empty((nb,), dtype=torch.uint8, device=X.device) if nb else None
        made.append(workspace)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
    _on_stream(stream, *made)
    wp, wn = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    s = load().kq_lowrank_down(_ptr(X), _ptr(L1), M, K, r, _ptr(T), wp, wn, _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_lowrank_down")
    return T


def transform_quantize_lowrank(X, xform, L1, center=False, codes=None, scales=None, mu=None, T=None, workspace=None,
                               stream=None):
    """One pass over X: MXFP4 codes and scales of the (optionally centred, RPBH only)
    block-transformed X and the low-rank down-projection T = fp16(X L1^T).
    Returns (codes, scales, mu or None, T)."""
    torch = _torch()
    _check(X, "X", torch.float16)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M, K]")
    M, K = X.shape
    r = L1.shape[0]
    _check(L1, "L1", torch.float16, (r, K))
    dev = X.device
    made = []
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        made.append(codes)
    _check(codes, "codes", torch.uint8, (M, K // 2))
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        made.append(scales)
    _check(scales, "scales", torch.uint8, (M, K // 32))
    if center:
        if mu is None:
            mu = torch.empty((M,), dtype=torch.float16, device=dev)
            made.append(mu)
        _check(mu, "mu", torch.float16, (M,))
    else:
        mu = None
    if T is None:
        T = torch.empty((M, r), dtype=torch.float16, device=dev)
        made.append(T)
    _check(T, "T", torch.float16, (M, r))
    if workspace is None:
        nb = lowrank_down_workspace_bytes(M, K, r)
        workspace = torch.empty((nb,), dtype=torch.uint8, device=dev) if nb else None
        made.append(workspace)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
    _on_stream(stream, *made)
    wp, wn = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    s = load().kq_transform_quantize_lowrank(xform.c(), int(bool(center)), _ptr(X), M, K, _ptr(codes), _ptr(scales),
                                             _ptr(mu), _ptr(L1), r, _ptr(T), wp, wn, _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_transform_quantize_lowrank")
    return codes, scales, mu, T


def svd_lowrank_workspace_bytes(N, K, r, l):
    return int(load().kq_svd_lowrank_workspace_bytes(N, K, r, l))


def svd_lowrank(W, r, omega, iters=4, L1=None, L2=None, R=None, sigma=None, workspace=None, stream=None):
    """Offline rank-r extraction: W (fp16 [N][K]) ~ L2 L1 + R.  omega: float32 [K][l]
    device starting block (l > r).  Returns (L1 [r][K], L2 [N][r], R [N][K], sigma [r])."""
    torch = _torch()
    _check(W, "W", torch.float16)
    N, K = W.shape
    _check(omega, "omega", torch.float32)
    if omega.dim() != 2 or omega.shape[0] != K:
        raise ValueError("omega must be [K, l]")
    l = omega.shape[1]
    dev = W.device
    made = []

    def _new(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=dev)
        made.append(t)
        return t
    L1 = _new((r, K), torch.float16) if L1 is None else L1
    L2 = _new((N, r), torch.float16) if L2 is None else L2
    R = _new((N, K), torch.float16) if R is None else R
    sigma = _new((r,), torch.float32) if sigma is None else sigma
    _check(L1, "L1", torch.float16, (r, K))
    _check(L2, "L2", torch.float16, (N, r))
    _check(R, "R", torch.float16, (N, K))
    _check(sigma, "sigma", torch.float32, (r,))
    nb = svd_lowrank_workspace_bytes(N, K, r, l)
    if workspace is None:
        workspace = _new((max(nb, 256),), torch.uint8)
    _check(workspace, "workspace", torch.uint8)
    _on_stream(stream, *made)
    s = load().kq_svd_lowrank(_ptr(W), N, K, r, _ptr(omega), l, int(iters), _ptr(L1), _ptr(L2), _ptr(R),
                              _ptr(sigma), _ptr(workspace), workspace.numel(), _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_svd_lowrank")
    return L1, L2, R, sigma


def _linear_operands(xcodes, xscales, wcodes, wscales, fmt):
    torch = _torch()
    f = _FMT[fmt]
    _check(xcodes, "xcodes", torch.uint8)
    M = xcodes.shape[0]
    K = xcodes.shape[1] * 2
    N = wcodes.shape[0]
    _check(wcodes, "wcodes", torch.uint8, (N, K // 2) if f == FMT_MXFP4 else (N, K // 4))
    if f == FMT_MXFP4:
        _check(xscales, "xscales", torch.uint8, (M, K // 32))
        _check(wscales, "wscales", torch.uint8, (N, K // 32))
    else:
        _check(xscales, "xscales", torch.float32, (M,))
        _check(wscales, "wscales", torch.float16, (N, K // 32))
    return f, M, K, N


def _linear_tail(M, N, mu, wbar, Y, dev):
    torch = _torch()
    if mu is not None:
        _check(mu, "mu", torch.float16, (M,))
        _check(wbar, "wbar", torch.float16, (N,))
    made = Y is None
    Y = torch.empty((M, N), dtype=torch.float16, device=dev) if Y is None else Y
    _check(Y, "Y", torch.float16, (M, N))
    return Y, made


def w4a4_linear_workspace_bytes(M, r):
    """Workspace bytes kq_w4a4_linear needs for M tokens and rank r (0 when r == 0)."""
    return int(load().kq_w4a4_linear_workspace_bytes(M, r))


def w4a4_linear(xcodes, xscales, wcodes, wscales, X=None, L1=None, L2=None, mu=None, wbar=None,
                fmt="mxfp4", Y=None, workspace=None, stream=None):
    """Y = Xq Wq^T + (X L1^T) L2^T + mu wbar^T (fp16 [M][N]): the down-projection of the
    low-rank branch runs inside the call (its result held in the workspace).  X fp16
    [M][K], L1 fp16 [r][K], L2 fp16 [N][r].  workspace: a uint8 device tensor of at least
    w4a4_linear_workspace_bytes(M, r) bytes (256-byte aligned); by default one is taken
    from torch's allocator.  fmt 'mxfp4' (W4A4) or 'lm2' (W2A4, no branches)."""
    torch = _torch()
    f, M, K, N = _linear_operands(xcodes, xscales, wcodes, wscales, fmt)
    r = 0
    if L1 is not None:
        r = L1.shape[0]
        _check(X, "X", torch.float16, (M, K))
        _check(L1, "L1", torch.float16, (r, K))
        _check(L2, "L2", torch.float16, (N, r))
    Y, made_y = _linear_tail(M, N, mu, wbar, Y, xcodes.device)
    made = [Y] if made_y else []
    if r and workspace is None:
        workspace = torch.empty((w4a4_linear_workspace_bytes(M, r),), dtype=torch.uint8, device=xcodes.device)
        made.append(workspace)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
    _on_stream(stream, *made)
    wp, wn = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    s = load().kq_w4a4_linear(f, _ptr(xcodes), _ptr(xscales), M, K, _ptr(wcodes), _ptr(wscales), N,
                              _ptr(X if r else None), _ptr(L1 if r else None), _ptr(L2 if r else None), r,
                              _ptr(mu), _ptr(wbar), _ptr(Y), wp, wn, _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_w4a4_linear")
    return Y


def w4a4_linear_t(xcodes, xscales, wcodes, wscales, T=None, L2=None, mu=None, wbar=None,
                  fmt="mxfp4", Y=None, stream=None):
    """Y = Xq Wq^T + T L2^T + mu wbar^T (fp16 [M][N]) with the down-projection T (fp16
    [M][r]) already computed.  fmt 'mxfp4' (W4A4) or 'lm2' (W2A4)."""
    torch = _torch()
    f, M, K, N = _linear_operands(xcodes, xscales, wcodes, wscales, fmt)
    r = 0
    if T is not None:
        r = T.shape[1]
        _check(T, "T", torch.float16, (M, r))
        _check(L2, "L2", torch.float16, (N, r))
    Y, made_y = _linear_tail(M, N, mu, wbar, Y, xcodes.device)
    if made_y:
        _on_stream(stream, Y)
    s = load().kq_w4a4_linear_t(f, _ptr(xcodes), _ptr(xscales), M, K, _ptr(wcodes), _ptr(wscales), N,
                                _ptr(T), _ptr(L2 if r else None), r, _ptr(mu), _ptr(wbar), _ptr(Y),
                                _stream(stream))
    if s != KQ_OK:
        raise KQError(s, "kq_w4a4_linear_t")
    return Y
