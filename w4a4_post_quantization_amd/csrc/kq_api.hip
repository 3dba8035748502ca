// C ABI of libkq: host-side argument validation and dispatch to the kernels.
#include <cmath>
#include <cstring>
#include <mutex>

#include "kq.h"
#include "kq_launch.hpp"

namespace kq {

// ---- Lloyd-Max codebooks (OrbitQuant §03: one fixed codebook for the rotated,
// approximately Gaussian coordinates).  Symmetric n-level quantizer for N(0, 1): Lloyd's
// fixed point, levels = conditional means of their cells, thresholds = midpoints.
static double npdf(double t) { return std::exp(-0.5 * t * t) * 0.39894228040143267794; }
// P(a < Z < b) for 0 <= a < b <= inf, through erfc so the upper tail keeps its accuracy
static double nmass(double a, double b) {
  const double ua = 0.5 * std::erfc(a * 0.70710678118654752440);
  const double ub = std::isinf(b) ? 0.0 : 0.5 * std::erfc(b * 0.70710678118654752440);
  return ua - ub;
}

bool lloyd_max_levels(int n, double* out) {
  if (n != 4 && n != 16) return false;
  const int h = n / 2;
  double lv[8], nx[8];
  for (int i = 0; i < h; ++i) lv[i] = 3.0 * (i + 0.5) / h;  // any increasing start converges
  for (int it = 0; it < 200000; ++it) {
    double diff = 0.0;
    for (int i = 0; i < h; ++i) {
      const double lo = i == 0 ? 0.0 : 0.5 * (lv[i - 1] + lv[i]);
      const double hi = i == h - 1 ? INFINITY : 0.5 * (lv[i] + lv[i + 1]);
      const double num = npdf(lo) - (std::isinf(hi) ? 0.0 : npdf(hi));
      nx[i] = num / nmass(lo, hi);
      diff = std::fmax(diff, std::fabs(nx[i] - lv[i]));
    }
    for (int i = 0; i < h; ++i) lv[i] = nx[i];
    if (diff <= 1e-15) break;
  }
  for (int i = 0; i < h; ++i) out[i] = lv[i];
  return true;
}

const LmTables& lm_tables() {
  static LmTables t;
  static std::once_flag once;
  std::call_once(once, [] {
    double l16[8], l4[2];
    lloyd_max_levels(16, l16);
    lloyd_max_levels(4, l4);
    for (int i = 0; i < 8; ++i) t.l16[i] = (float)l16[i];
    for (int i = 0; i < 7; ++i) t.t16[i] = (float)(0.5 * (l16[i] + l16[i + 1]));
    t.l4[0] = (float)l4[0];
    t.l4[1] = (float)l4[1];
    t.t4 = (float)(0.5 * (l4[0] + l4[1]));
  });
  return t;
}

// inverse of a small row-major matrix by Gauss-Jordan with partial pivoting (double)
static bool invert(const float* a, int n, float* out) {
  double m[8][16];
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < 2 * n; ++j) m[i][j] = j < n ? (double)a[i * n + j] : (j - n == i ? 1.0 : 0.0);
  double scale = 0.0;
  for (int i = 0; i < n * n; ++i) {
    if (!std::isfinite(a[i])) return false;
    scale = std::fmax(scale, std::fabs((double)a[i]));
  }
  if (scale == 0.0) return false;
  for (int c = 0; c < n; ++c) {
    int p = c;
    for (int i = c + 1; i < n; ++i)
      if (std::fabs(m[i][c]) > std::fabs(m[p][c])) p = i;
    if (std::fabs(m[p][c]) <= 1e-12 * scale) return false;
    if (p != c)
      for (int j = 0; j < 2 * n; ++j) std::swap(m[p][j], m[c][j]);
    const double d = m[c][c];
    for (int j = 0; j < 2 * n; ++j) m[c][j] /= d;
    for (int i = 0; i < n; ++i) {
      if (i == c) continue;
      const double f = m[i][c];
      if (f != 0.0)
        for (int j = 0; j < 2 * n; ++j) m[i][j] -= f * m[c][j];
    }
  }
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) out[i * n + j] = (float)m[i][n + j];
  return true;
}

}  // namespace kq

using namespace kq;

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static kq_status hip_status(hipError_t e) { return e == hipSuccess ? KQ_OK : KQ_ERR_HIP; }

static kq_status check_xform(const kq_xform* xf, int64_t K) {
  if (!xf) return KQ_ERR_NULL;
  if (xf->kind < KQ_XFORM_NONE || xf->kind > KQ_XFORM_KRON_4X8_BLOCKS || xf->reserved != 0) return KQ_ERR_UNSUPPORTED;
  if (xf->K != K) return KQ_ERR_SHAPE;
  if (xf->kind == KQ_XFORM_RPBH_32) {
    if (!xf->perm || !xf->sign) return KQ_ERR_NULL;
    if (!aligned(xf->perm, 16) || !aligned(xf->sign, 4)) return KQ_ERR_ALIGN;
  }
  if (xf->kind == KQ_XFORM_DENSE_32) {
    if (!xf->P) return KQ_ERR_NULL;
    if (!aligned(xf->P, 16)) return KQ_ERR_ALIGN;
  }
  if (xf->kind == KQ_XFORM_KRON_4X8_BLOCKS) {
    if (!xf->AB) return KQ_ERR_NULL;
    if (!aligned(xf->AB, 16)) return KQ_ERR_ALIGN;
  }
  if (xf->pts) {
    if (xf->kind == KQ_XFORM_RPBH_32) return KQ_ERR_UNSUPPORTED;
    if (!aligned(xf->pts, 16)) return KQ_ERR_ALIGN;
  }
  if (xf->kind == KQ_XFORM_KRON_4X8) {
    for (int i = 0; i < 16; ++i)
      if (!std::isfinite(xf->A[i])) return KQ_ERR_VALUE;
    for (int i = 0; i < 64; ++i)
      if (!std::isfinite(xf->B[i])) return KQ_ERR_VALUE;
  }
  return KQ_OK;
}

extern "C" {

int32_t kq_abi_version(void) { return KQ_ABI_VERSION; }

const char* kq_status_str(kq_status s) {
  switch (s) {
    case KQ_OK: return "KQ_OK";
    case KQ_ERR_NULL: return "KQ_ERR_NULL: a required pointer is NULL";
    case KQ_ERR_SHAPE: return "KQ_ERR_SHAPE: invalid shape (M, N >= 1, K % 32 == 0, descriptor K, rank)";
    case KQ_ERR_ALIGN: return "KQ_ERR_ALIGN: a device pointer is not suitably aligned";
    case KQ_ERR_UNSUPPORTED: return "KQ_ERR_UNSUPPORTED: unknown enum or size outside the supported range";
    case KQ_ERR_VALUE: return "KQ_ERR_VALUE: transform factor singular or not finite";
    case KQ_ERR_HIP: return "KQ_ERR_HIP: a HIP launch failed";
    case KQ_ERR_WORKSPACE: return "KQ_ERR_WORKSPACE: workspace missing or smaller than the call needs";
    default: return "KQ_ERR_UNKNOWN: unknown status code";
  }
}

kq_status kq_lloyd_max_levels(int32_t n, double* levels_out) {
  if (!levels_out) return KQ_ERR_NULL;
  return lloyd_max_levels(n, levels_out) ? KQ_OK : KQ_ERR_UNSUPPORTED;
}

kq_status kq_clock_probe(int32_t spin_us, uint64_t* out, hipStream_t stream) {
  if (!out) return KQ_ERR_NULL;
  if (spin_us < 1 || spin_us > 1000000) return KQ_ERR_UNSUPPORTED;
  if (!aligned(out, 8)) return KQ_ERR_ALIGN;
  return hip_status(launch_clock_probe(spin_us, out, stream));
}

kq_status kq_mfma_fp4_probe(int32_t iters, int32_t workgroups, const void* codes, float* out, hipStream_t stream) {
  if (!codes || !out) return KQ_ERR_NULL;
  if (iters < 1 || iters > 1000000 || workgroups < 1 || workgroups > 65536) return KQ_ERR_UNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(out, 4)) return KQ_ERR_ALIGN;
  return hip_status(launch_mfma_fp4_probe(iters, workgroups, codes, out, stream));
}

kq_status kq_transform_quantize(const kq_xform* xf, int32_t fmt, int32_t center, const void* X, int64_t M,
                                int64_t K, uint8_t* codes, void* scales, void* mu, hipStream_t stream) {
  if (!X || !codes || !scales) return KQ_ERR_NULL;
  if (center && !mu) return KQ_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0) return KQ_ERR_SHAPE;
  if (fmt != KQ_FMT_MXFP4 && fmt != KQ_FMT_LM4_TOKEN) return KQ_ERR_UNSUPPORTED;
  kq_status st = check_xform(xf, K);
  if (st != KQ_OK) return st;
  if (!aligned(X, 16) || !aligned(codes, 16)) return KQ_ERR_ALIGN;
  if (fmt == KQ_FMT_LM4_TOKEN && !aligned(scales, 4)) return KQ_ERR_ALIGN;
  if (center && !aligned(mu, 2)) return KQ_ERR_ALIGN;
  KronFactors f;
  std::memcpy(f.A, xf->A, sizeof f.A);
  std::memcpy(f.B, xf->B, sizeof f.B);
  // MXFP4 goes through the matrix-core transforms (streaming for Kronecker / identity
  // without centring, row-staged for RPBH), and so does RPBH with the per-token Lloyd-Max
  // format without centring; the other Lloyd-Max cases and centred Kronecker / identity
  // use the row-staged vector kernel.
  // A dense P, per-block factors and power-of-two channel scaling run on the matrix-core
  // stream paths only (MXFP4, no centring).
  const bool mx = fmt == KQ_FMT_MXFP4;
  const bool stream_path = mx && !center && xf->kind != KQ_XFORM_RPBH_32;
  const bool rpbh_mfma = mx && xf->kind == KQ_XFORM_RPBH_32;
  if ((xf->kind == KQ_XFORM_DENSE_32 || xf->kind == KQ_XFORM_KRON_4X8_BLOCKS || xf->pts) && !stream_path)
    return KQ_ERR_UNSUPPORTED;
  if (!stream_path && K > 16384) return KQ_ERR_UNSUPPORTED;
  hipError_t e;
  if (stream_path && xf->kind == KQ_XFORM_KRON_4X8_BLOCKS) {
    e = launch_kron_blocks_mx(static_cast<const __half*>(X), M, K, xf->AB, xf->pts, codes,
                              static_cast<uint8_t*>(scales), stream);
  } else if (stream_path) {
    e = launch_kron_mx_mfma(xf->kind, static_cast<const __half*>(X), M * (K / 32), f, xf->P, xf->pts, K / 32,
                            codes, static_cast<uint8_t*>(scales), stream);
  } else if (xf->kind == KQ_XFORM_RPBH_32 && fmt == KQ_FMT_LM4_TOKEN && !center) {
    e = launch_rpbh_lm4_mfma(static_cast<const __half*>(X), M, K, xf->perm, xf->sign, codes,
                             static_cast<float*>(scales), stream);
  } else if (rpbh_mfma) {
    e = launch_rpbh_mx_mfma(center != 0, static_cast<const __half*>(X), M, K, xf->perm, xf->sign, codes,
                            static_cast<uint8_t*>(scales), static_cast<__half*>(mu), stream);
  } else {
    e = launch_row_quant(xf->kind, mx ? 0 : 1, center != 0, static_cast<const __half*>(X), M, K, f, xf->perm,
                         xf->sign, codes, scales, static_cast<__half*>(mu), stream);
  }
  return hip_status(e);
}

static kq_status fold(const kq_xform* xf, int32_t fmt, bool kn, const void* W, int64_t N, int64_t K,
                      uint8_t* wcodes, void* wscales, void* wbar, hipStream_t stream) {
  if (!W || !wcodes || !wscales) return KQ_ERR_NULL;
  if (N < 1 || K < 32 || K % 32 != 0) return KQ_ERR_SHAPE;
  if (fmt != KQ_FMT_MXFP4 && fmt != KQ_FMT_LM2_G32) return KQ_ERR_UNSUPPORTED;
  kq_status st = check_xform(xf, K);
  if (st != KQ_OK) return st;
  if (!aligned(W, 16) || !aligned(wcodes, 16)) return KQ_ERR_ALIGN;
  if (fmt == KQ_FMT_LM2_G32 && !aligned(wscales, 2)) return KQ_ERR_ALIGN;
  if (wbar && !aligned(wbar, 2)) return KQ_ERR_ALIGN;
  KronFactors finv;
  std::memset(&finv, 0, sizeof finv);
  if (xf->kind == KQ_XFORM_KRON_4X8) {
    if (!invert(xf->A, 4, finv.A) || !invert(xf->B, 8, finv.B)) return KQ_ERR_VALUE;
  }
  hipError_t e = launch_fold(xf->kind, fmt == KQ_FMT_MXFP4 ? 0 : 2, kn, static_cast<const __half*>(W), N, K, finv,
                             xf->perm, xf->sign, xf->kind == KQ_XFORM_KRON_4X8_BLOCKS ? xf->AB : xf->P, xf->pts,
                             wcodes, wscales, stream);
  if (e != hipSuccess) return KQ_ERR_HIP;
  if (wbar) e = launch_colsum(kn, static_cast<const __half*>(W), N, K, static_cast<__half*>(wbar), stream);
  return hip_status(e);
}

kq_status kq_fold_inverse_into_weights(const kq_xform* xf, int32_t fmt, const void* W, int64_t K, int64_t N,
                                       uint8_t* wcodes, void* wscales, void* wbar, hipStream_t stream) {
  return fold(xf, fmt, true, W, N, K, wcodes, wscales, wbar, stream);
}

kq_status kq_fold_inverse_into_weights_nk(const kq_xform* xf, int32_t fmt, const void* Wt, int64_t N, int64_t K,
                                          uint8_t* wcodes, void* wscales, void* wbar, hipStream_t stream) {
  return fold(xf, fmt, false, Wt, N, K, wcodes, wscales, wbar, stream);
}

static bool lr_rank(int32_t r) { return r == 16 || r == 32 || r == 48 || r == 64; }

size_t kq_lowrank_down_workspace_bytes(int64_t M, int64_t K, int32_t r) {
  if (M < 1 || K < 32 || K % 32 != 0 || !lr_rank(r)) return 0;
  return lowrank_workspace_bytes(M, K, r);
}

kq_status kq_lowrank_down(const void* X, const void* L1, int64_t M, int64_t K, int32_t r, void* T,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!X || !L1 || !T) return KQ_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0) return KQ_ERR_SHAPE;
  if (!lr_rank(r)) return KQ_ERR_SHAPE;
  if (M > (1LL << 31) - 64 || K > (1LL << 20)) return KQ_ERR_UNSUPPORTED;
  if (!aligned(X, 16) || !aligned(L1, 16) || !aligned(T, 16)) return KQ_ERR_ALIGN;
  if (workspace_bytes && !workspace) return KQ_ERR_NULL;
  if (workspace && !aligned(workspace, 16)) return KQ_ERR_ALIGN;
  return hip_status(launch_lowrank_down(static_cast<const __half*>(X), static_cast<const __half*>(L1), M, K, r,
                                        static_cast<__half*>(T), static_cast<float*>(workspace),
                                        workspace ? workspace_bytes : 0, stream));
}

kq_status kq_transform_quantize_lowrank(const kq_xform* xf, int32_t center, const void* X, int64_t M, int64_t K,
                                        uint8_t* codes, void* scales, void* mu, const void* L1, int32_t r, void* T,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!X || !codes || !scales || !L1 || !T) return KQ_ERR_NULL;
  if (center && !mu) return KQ_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0) return KQ_ERR_SHAPE;
  if (!lr_rank(r)) return KQ_ERR_SHAPE;
  kq_status st = check_xform(xf, K);
  if (st != KQ_OK) return st;
  const bool rpbh = xf->kind == KQ_XFORM_RPBH_32;
  if (!rpbh && xf->kind != KQ_XFORM_NONE && xf->kind != KQ_XFORM_KRON_4X8 && xf->kind != KQ_XFORM_DENSE_32)
    return KQ_ERR_UNSUPPORTED;
  if (xf->pts) return KQ_ERR_UNSUPPORTED;
  if (center && !rpbh) return KQ_ERR_UNSUPPORTED;
  if (rpbh && K > 16384) return KQ_ERR_UNSUPPORTED;
  if (M > (1LL << 31) - 64 || K > (1LL << 20)) return KQ_ERR_UNSUPPORTED;
  if (!aligned(X, 16) || !aligned(L1, 16) || !aligned(T, 16) || !aligned(codes, 16)) return KQ_ERR_ALIGN;
  if (center && !aligned(mu, 2)) return KQ_ERR_ALIGN;
  if (workspace_bytes && !workspace) return KQ_ERR_NULL;
  if (workspace && !aligned(workspace, 16)) return KQ_ERR_ALIGN;
  const __half* Xh = static_cast<const __half*>(X);
  __half* Th = static_cast<__half*>(T);
  if (rpbh) {
    // the permutation spans the whole row, so the quantizer stages full rows while the
    // projection streams k-chunks of 64-row blocks: the transform, then the split-K
    // down-projection (two launches; X is read twice)
    hipError_t e = launch_rpbh_mx_mfma(center != 0, Xh, M, K, xf->perm, xf->sign, codes, static_cast<uint8_t*>(scales),
                                       static_cast<__half*>(mu), stream);
    if (e != hipSuccess) return KQ_ERR_HIP;
    return hip_status(launch_lowrank_down(Xh, static_cast<const __half*>(L1), M, K, r, Th,
                                          static_cast<float*>(workspace), workspace ? workspace_bytes : 0, stream));
  }
  KronFactors f;
  std::memcpy(f.A, xf->A, sizeof f.A);
  std::memcpy(f.B, xf->B, sizeof f.B);
  return hip_status(launch_lowrank_xform_mx(xf->kind, Xh, static_cast<const __half*>(L1), M, K, r, Th,
                                            static_cast<float*>(workspace), workspace ? workspace_bytes : 0, f, xf->P,
                                            codes, static_cast<uint8_t*>(scales), stream));
}

size_t kq_svd_lowrank_workspace_bytes(int64_t N, int64_t K, int32_t r, int32_t l) {
  if (N < 1 || K < 32 || K % 32 != 0 || (r != 16 && r != 32 && r != 64) || l <= r || l > 96) return 0;
  return svd_workspace_bytes(N, K, l, r);
}

kq_status kq_svd_lowrank(const void* W, int64_t N, int64_t K, int32_t r, const float* omega, int32_t l,
                         int32_t iters, void* L1, void* L2, void* R, float* sigma, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!W || !omega || !L1 || !L2 || !R || !workspace) return KQ_ERR_NULL;
  if (N < 1 || K < 32 || K % 32 != 0) return KQ_ERR_SHAPE;
  if (r != 16 && r != 32 && r != 64) return KQ_ERR_SHAPE;
  if (l <= r || l > 96 || l > N || l > K || iters < 0 || iters > 16) return KQ_ERR_SHAPE;
  if (N > (1LL << 20) || K > (1LL << 20)) return KQ_ERR_UNSUPPORTED;
  if (workspace_bytes < svd_workspace_bytes(N, K, l, r)) return KQ_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(omega, 16) || !aligned(L1, 16) || !aligned(L2, 16) || !aligned(R, 16) ||
      !aligned(workspace, 256) || (sigma && !aligned(sigma, 4)))
    return KQ_ERR_ALIGN;
  return hip_status(launch_svd_lowrank(static_cast<const __half*>(W), N, K, r, omega, l, iters,
                                       static_cast<__half*>(L1), static_cast<__half*>(L2), static_cast<__half*>(R),
                                       sigma, workspace, stream));
}

// ---- Scratch of the allocation-free linear (kq_w4a4_linear_noalloc): a file-scope device
// array that holds T and the down-projection's split-K partial sums.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[KQ_NOALLOC_SCRATCH_BYTES];

static void* scratch_device_ptr(int dev) {
  constexpr int kMaxDevices = 64;
  static std::mutex mtx;
  static void* ptrs[kMaxDevices] = {};
  static bool done[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mtx);
  if (!done[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
    done[dev] = true;
  }
  return ptrs[dev];
}

// Arguments of the 4-bit product and its epilogue, shared by both linear forms (the
// low-rank operands are checked by the callers).
static kq_status check_linear(int32_t fmt, const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                              const uint8_t* wcodes, const void* wscales, int64_t N, int32_t r, const void* mu,
                              const void* wbar, const void* Y) {
  if (!xcodes || !xscales || !wcodes || !wscales || !Y) return KQ_ERR_NULL;
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0) return KQ_ERR_SHAPE;
  if (r != 0 && !lr_rank(r)) return KQ_ERR_SHAPE;
  if ((mu == nullptr) != (wbar == nullptr)) return KQ_ERR_SHAPE;
  if (M > (1LL << 30) || N > (1LL << 20) || K > (1LL << 20)) return KQ_ERR_UNSUPPORTED;
  if (N % 16 != 0) return KQ_ERR_UNSUPPORTED;
  if (fmt == KQ_FMT_MXFP4) {
    if (K % 128 != 0) return KQ_ERR_UNSUPPORTED;
  } else if (fmt == KQ_FMT_LM2_G32) {
    if (r != 0 || mu) return KQ_ERR_UNSUPPORTED;
  } else {
    return KQ_ERR_UNSUPPORTED;
  }
  if (!aligned(xcodes, 16) || !aligned(wcodes, 16) || !aligned(Y, 16)) return KQ_ERR_ALIGN;
  if (!aligned(xscales, 4) || !aligned(wscales, 4)) return KQ_ERR_ALIGN;
  if (mu && (!aligned(mu, 2) || !aligned(wbar, 16))) return KQ_ERR_ALIGN;
  return KQ_OK;
}

static hipError_t run_linear(int32_t fmt, const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                             const uint8_t* wcodes, const void* wscales, int64_t N, const void* T, const void* L2,
                             int32_t r, const void* mu, const void* wbar, void* Y, hipStream_t stream) {
  if (fmt == KQ_FMT_MXFP4)
    return launch_w4a4_gemm(xcodes, static_cast<const uint8_t*>(xscales), M, K, wcodes,
                            static_cast<const uint8_t*>(wscales), N, r ? static_cast<const __half*>(T) : nullptr,
                            static_cast<const __half*>(L2), r, static_cast<const __half*>(mu),
                            static_cast<const __half*>(wbar), static_cast<__half*>(Y), stream);
  return launch_w2a4_gemm(xcodes, static_cast<const float*>(xscales), M, K, wcodes,
                          static_cast<const __half*>(wscales), N, static_cast<__half*>(Y), stream);
}

size_t kq_w4a4_linear_workspace_bytes(int64_t M, int32_t r) {
  if (M < 1 || M > (1LL << 30) || (r != 0 && !lr_rank(r))) return 0;
  return lowrank_linear_workspace_bytes(M, r);
}

kq_status kq_w4a4_linear(int32_t fmt, const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                         const uint8_t* wcodes, const void* wscales, int64_t N, const void* X, const void* L1,
                         const void* L2, int32_t r, const void* mu, const void* wbar, void* Y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  kq_status st = check_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, r, mu, wbar, Y);
  if (st != KQ_OK) return st;
  if (r > 0) {
    if (!X || !L1 || !L2) return KQ_ERR_NULL;
    if (!aligned(X, 16) || !aligned(L1, 16) || !aligned(L2, 16)) return KQ_ERR_ALIGN;
    const size_t tb = lowrank_t_bytes(M, r);
    if (!workspace || workspace_bytes < lowrank_linear_workspace_bytes(M, r)) return KQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KQ_ERR_ALIGN;
    __half* T = static_cast<__half*>(workspace);
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + tb);
    hipError_t e = launch_lowrank_down(static_cast<const __half*>(X), static_cast<const __half*>(L1), M, K, r, T, part,
                                       workspace_bytes - tb, stream);
    if (e != hipSuccess) return KQ_ERR_HIP;
    return hip_status(run_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, stream));
  }
  return hip_status(run_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, nullptr, nullptr, 0, mu, wbar, Y,
                               stream));
}

kq_status kq_w4a4_linear_noalloc(int32_t fmt, const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                                 const uint8_t* wcodes, const void* wscales, int64_t N, const void* X,
                                 const void* L1, const void* L2, int32_t r, const void* mu, const void* wbar, void* Y,
                                 hipStream_t stream) {
  kq_status st = check_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, r, mu, wbar, Y);
  if (st != KQ_OK) return st;
  if (r == 0)
    return hip_status(run_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, nullptr, nullptr, 0, mu, wbar, Y,
                                 stream));
  if (!X || !L1 || !L2) return KQ_ERR_NULL;
  if (!aligned(X, 16) || !aligned(L1, 16) || !aligned(L2, 16)) return KQ_ERR_ALIGN;
  const size_t tb = lowrank_t_bytes(M, r);
  if (tb > KQ_NOALLOC_SCRATCH_BYTES) return KQ_ERR_WORKSPACE;   // T alone would not fit the scratch
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
  uint8_t* base = static_cast<uint8_t*>(scratch_device_ptr(dev));
  if (!base) return KQ_ERR_HIP;
  // T first, then as many split-K slices of partial sums as the rest holds (fewer slices
  // than the workspace form would take only when the scratch is the limit; every slice and
  // T are written in full before they are read, so nothing needs clearing)
  __half* T = reinterpret_cast<__half*>(base);
  float* part = reinterpret_cast<float*>(base + tb);
  hipError_t e = launch_lowrank_down(static_cast<const __half*>(X), static_cast<const __half*>(L1), M, K, r, T, part,
                                     KQ_NOALLOC_SCRATCH_BYTES - tb, stream);
  if (e != hipSuccess) return KQ_ERR_HIP;
  return hip_status(run_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, stream));
}

kq_status kq_w4a4_linear_t(int32_t fmt, const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                           const uint8_t* wcodes, const void* wscales, int64_t N, const void* T, const void* L2,
                           int32_t r, const void* mu, const void* wbar, void* Y, hipStream_t stream) {
  kq_status st = check_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, r, mu, wbar, Y);
  if (st != KQ_OK) return st;
  if (r > 0) {
    if (!T || !L2) return KQ_ERR_NULL;
    if (!aligned(T, 16) || !aligned(L2, 16)) return KQ_ERR_ALIGN;
  }
  return hip_status(run_linear(fmt, xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, stream));
}

}  // extern "C"
