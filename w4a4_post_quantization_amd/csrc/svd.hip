// Offline low-rank extraction for the 16-bit branch (SVDQuant explainer §3: the weight is
// split into a low-rank part kept in 16 bits and a residual that is quantized to 4 bits,
// the low-rank part being the leading singular directions).  Runs once per layer, outside
// the timed path; written for clarity.
//
// With W given as Wt [N][K] (row n = output n), the rank-r part is L2 L1 with
// L2 = U_r S_r^1/2 [N][r] and L1 = S_r^1/2 V_r^T [r][K] (an even split of the singular
// values, so both factors have the same scale in fp16), and the residual is
// R = fp16(Wt - L2 L1) computed with the fp16 factors the branch will use, so that
// X R^T + (X L1^T) L2^T reproduces X Wt^T up to the 4-bit quantization of R.
//
// The leading subspace comes from randomized subspace iteration with l = r + oversampling
// columns (Halko, Martinsson and Tropp, 2011, algorithms 4.4 and 5.1): Y = Wt Omega, then
// `iters` times Z = Wt^T Y and Y = Wt Z, each product re-orthonormalized (CholeskyQR2:
// Gram matrix in float64, Cholesky and triangular inverse on one workgroup, Y <- Y R^-1,
// twice); then B = Y^T Wt, the eigen-decomposition of B B^T by cyclic Jacobi in float64,
// and the factors from its leading r eigenpairs.  Products are float32.
#include "kq_device.hpp"
#include "kq_launch.hpp"

#include <algorithm>

namespace kq {

constexpr int SVD_LMAX = 96;

// C(i, j) = sum_p A(i, p) B(p, j), i < m, j < n, p < k, with A(i, p) = A[i as + p ap] and
// B(p, j) = B[p bs + j bp] (TA, TB: float or __half), float32 accumulation.
// EPI 0: C float [i cs + j]; 1: C __half; 2: C __half = fp16(D[i cs + j] - acc).
// 64x64 tiles, k-chunks of 16 through LDS, 4x4 outputs per thread.
template <typename TA, typename TB, int EPI>
__global__ __launch_bounds__(256) void svd_gemm_kernel(const TA* __restrict__ A, int64_t as, int64_t ap,
                                                       const TB* __restrict__ B, int64_t bs, int64_t bp,
                                                       void* __restrict__ C, int64_t cs, const __half* __restrict__ D,
                                                       int64_t m, int64_t n, int64_t k) {
  __shared__ float sa[16][65];
  __shared__ float sb[16][65];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  float acc[4][4] = {};
  for (int64_t p0 = 0; p0 < k; p0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = t + 256 * e, ii = idx >> 4, pp = idx & 15;      // A tile: 64 rows x 16
      const int64_t i = i0 + ii, p = p0 + pp;
      sa[pp][ii] = (i < m && p < k) ? (float)A[i * as + p * ap] : 0.0f;
      const int jj = idx & 63, qq = idx >> 6;                         // B tile: 16 x 64 columns
      const int64_t j = j0 + jj, pb = p0 + qq;
      sb[qq][jj] = (j < n && pb < k) ? (float)B[pb * bs + j * bp] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < 16; ++pp) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = sa[pp][ty + 16 * u];
#pragma unroll
      for (int v = 0; v < 4; ++v) b[v] = sb[pp][tx + 16 * v];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fmaf(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = i0 + ty + 16 * u, j = j0 + tx + 16 * v;
      if (i >= m || j >= n) continue;
      if (EPI == 0) static_cast<float*>(C)[i * cs + j] = acc[u][v];
      else if (EPI == 1) static_cast<__half*>(C)[i * cs + j] = __float2half_rn(acc[u][v]);
      else static_cast<__half*>(C)[i * cs + j] = __float2half_rn(__half2float(D[i * cs + j]) - acc[u][v]);
    }
}

// G[a][b] = sum_t V[t s0 + a s1] V[t s0 + b s1], t < T, in float64 (a, b < l).
__global__ __launch_bounds__(256) void svd_gram_kernel(const float* __restrict__ V, int64_t s0, int64_t s1,
                                                       int64_t T, int l, double* __restrict__ G) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= l * l) return;
  const int a = e / l, b = e % l;
  if (b < a) return;                                   // the upper triangle; mirrored below
  double acc = 0.0;
  for (int64_t t = 0; t < T; ++t) acc += (double)V[t * s0 + a * s1] * (double)V[t * s0 + b * s1];
  G[a * l + b] = acc;
  G[b * l + a] = acc;
}

// One workgroup: G = R^T R (Cholesky, R upper), then Rinv = R^-1 (float32 out, l x l,
// row-major).  A non-positive pivot (rank-deficient Y) is replaced by 1 and its row of R
// by zeros, which zeroes that column of Y R^-1 instead of dividing by zero.
__global__ __launch_bounds__(256) void svd_chol_inv_kernel(const double* __restrict__ G, int l,
                                                           float* __restrict__ Rinv) {
  __shared__ double R[SVD_LMAX][SVD_LMAX + 1];
  __shared__ double Ri[SVD_LMAX][SVD_LMAX + 1];
  const int t = threadIdx.x;
  for (int e = t; e < l * l; e += 256) R[e / l][e % l] = G[e];
  __syncthreads();
  const double gmax = R[0][0];
  for (int c = 0; c < l; ++c) {
    if (t == 0) {
      const double d = R[c][c];
      R[c][c] = d > 1e-24 * (gmax > 0.0 ? gmax : 1.0) ? sqrt(d) : -1.0;   // -1 marks a dropped pivot
    }
    __syncthreads();
    const double piv = R[c][c];
    for (int j = c + 1 + t; j < l; j += 256) R[c][j] = piv > 0.0 ? R[c][j] / piv : 0.0;
    __syncthreads();
    for (int e = t; e < l * l; e += 256) {              // trailing update of the upper part
      const int i = e / l, j = e % l;
      if (i > c && j >= i) R[i][j] -= R[c][i] * R[c][j];
    }
    __syncthreads();
  }
  // inverse of the upper-triangular R, column by column (back substitution), one column
  // per thread
  for (int j = t; j < l; j += 256) {
    for (int i = l - 1; i >= 0; --i) {
      double s = (i == j) ? 1.0 : 0.0;
      for (int p = i + 1; p <= j; ++p) s -= R[i][p] * Ri[p][j];
      const double d = R[i][i];
      Ri[i][j] = (i > j || d <= 0.0) ? 0.0 : s / d;
    }
  }
  __syncthreads();
  for (int e = t; e < l * l; e += 256) Rinv[e] = (float)Ri[e / l][e % l];
}

// One workgroup: eigen-decomposition of the symmetric S (l x l, float64) by cyclic Jacobi
// sweeps, then the factors' small matrices from the r largest eigenvalues lambda (the
// squared singular values of B):  M2 [l][r] = U_r diag(lambda^1/4),
// M1 [r][l] = diag(lambda^-1/4) U_r^T.  An eigenvalue at or below 1e-24 lambda_max gives
// zero columns (that direction stays in the residual).
__global__ __launch_bounds__(64) void svd_eig_kernel(const double* __restrict__ S, int l, int r,
                                                     float* __restrict__ M2, float* __restrict__ M1,
                                                     float* __restrict__ sigma) {
  __shared__ double a[SVD_LMAX][SVD_LMAX + 1];
  __shared__ double v[SVD_LMAX][SVD_LMAX + 1];
  __shared__ double cs[2];
  __shared__ int order[SVD_LMAX];
  const int t = threadIdx.x;
  for (int e = t; e < l * l; e += 64) {
    a[e / l][e % l] = S[e];
    v[e / l][e % l] = (e / l == e % l) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 30; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < l; ++i)
      for (int j = 0; j < l; ++j) (i == j ? diag : off) += a[i][j] * a[i][j];
    if (off <= 1e-30 * diag) break;                    // every thread sees the same sums
    for (int p = 0; p < l - 1; ++p)
      for (int q = p + 1; q < l; ++q) {
        if (t == 0) {
          const double apq = a[p][q];
          double c = 1.0, s = 0.0;
          if (fabs(apq) > 1e-300) {
            const double th = (a[q][q] - a[p][p]) / (2.0 * apq);
            const double tt = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(th * th + 1.0));
            c = 1.0 / sqrt(tt * tt + 1.0);
            s = tt * c;
          }
          cs[0] = c;
          cs[1] = s;
        }
        __syncthreads();
        const double c = cs[0], s = cs[1];
        if (s != 0.0) {
          for (int k = t; k < l; k += 64) {            // columns p, q of a and v
            const double akp = a[k][p], akq = a[k][q];
            a[k][p] = c * akp - s * akq;
            a[k][q] = s * akp + c * akq;
            const double vkp = v[k][p], vkq = v[k][q];
            v[k][p] = c * vkp - s * vkq;
            v[k][q] = s * vkp + c * vkq;
          }
          __syncthreads();
          for (int k = t; k < l; k += 64) {            // rows p, q of a
            const double apk = a[p][k], aqk = a[q][k];
            a[p][k] = c * apk - s * aqk;
            a[q][k] = s * apk + c * aqk;
          }
        }
        __syncthreads();
      }
  }
  if (t == 0) {                                        // eigenvalues in descending order
    for (int i = 0; i < l; ++i) order[i] = i;
    for (int i = 1; i < l; ++i)
      for (int j = i; j > 0 && a[order[j]][order[j]] > a[order[j - 1]][order[j - 1]]; --j) {
        const int x = order[j];
        order[j] = order[j - 1];
        order[j - 1] = x;
      }
  }
  __syncthreads();
  const double lmax = a[order[0]][order[0]];
  for (int e = t; e < l * r; e += 64) {
    const int i = e / r, c = e % r, col = order[c];
    const double lam = a[col][col];
    const bool keep = lam > 1e-24 * (lmax > 0.0 ? lmax : 1.0);
    M2[i * r + c] = keep ? (float)(v[i][col] * sqrt(sqrt(lam))) : 0.0f;
    M1[c * l + i] = keep ? (float)(v[i][col] / sqrt(sqrt(lam))) : 0.0f;
  }
  for (int c = t; c < r; c += 64) {
    const double lam = a[order[c]][order[c]];
    sigma[c] = lam > 0.0 ? (float)sqrt(lam) : 0.0f;
  }
}

namespace {

struct SvdWork {
  float *Y, *Z, *Bm, *Y2, *Z2, *Rinv, *M1, *M2, *sigma;
  double *G;
};

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t svd_layout(int64_t N, int64_t K, int l, int r, SvdWork* w, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return base ? base + o : nullptr; };
  char* y = take((size_t)N * l * 4);
  char* y2 = take((size_t)N * l * 4);
  char* z = take((size_t)K * l * 4);
  char* z2 = take((size_t)K * l * 4);
  char* bm = take((size_t)l * K * 4);
  char* g = take((size_t)l * l * 8);
  char* ri = take((size_t)l * l * 4);
  char* m1 = take((size_t)r * l * 4);
  char* m2 = take((size_t)l * r * 4);
  char* sg = take((size_t)r * 4);
  if (w) {
    w->Y = reinterpret_cast<float*>(y);
    w->Y2 = reinterpret_cast<float*>(y2);
    w->Z = reinterpret_cast<float*>(z);
    w->Z2 = reinterpret_cast<float*>(z2);
    w->Bm = reinterpret_cast<float*>(bm);
    w->G = reinterpret_cast<double*>(g);
    w->Rinv = reinterpret_cast<float*>(ri);
    w->M1 = reinterpret_cast<float*>(m1);
    w->M2 = reinterpret_cast<float*>(m2);
    w->sigma = reinterpret_cast<float*>(sg);
  }
  return off;
}

template <typename TA, typename TB, int EPI>
hipError_t gemm(const TA* A, int64_t as, int64_t ap, const TB* B, int64_t bs, int64_t bp, void* C, int64_t cs,
                const __half* D, int64_t m, int64_t n, int64_t k, hipStream_t s) {
  const dim3 g((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
  hipLaunchKernelGGL((svd_gemm_kernel<TA, TB, EPI>), g, dim3(256), 0, s, A, as, ap, B, bs, bp, C, cs, D, m, n, k);
  return hipGetLastError();
}

// V [T][l] (row-major, T rows) <- orthonormal columns spanning the same space, via tmp.
hipError_t orthonormalize(float* V, float* tmp, int64_t T, int l, SvdWork& w, hipStream_t s) {
  for (int pass = 0; pass < 2; ++pass) {
    hipLaunchKernelGGL(svd_gram_kernel, dim3((unsigned)((l * l + 255) / 256)), dim3(256), 0, s, V, (int64_t)l,
                       (int64_t)1, T, l, w.G);
    hipLaunchKernelGGL(svd_chol_inv_kernel, dim3(1), dim3(256), 0, s, w.G, l, w.Rinv);
    hipError_t e = gemm<float, float, 0>(V, l, 1, w.Rinv, l, 1, tmp, l, nullptr, T, l, l, s);
    if (e != hipSuccess) return e;
    e = hipMemcpyAsync(V, tmp, (size_t)T * l * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace

size_t svd_workspace_bytes(int64_t N, int64_t K, int l, int r) { return svd_layout(N, K, l, r, nullptr, nullptr); }

hipError_t launch_svd_lowrank(const __half* Wt, int64_t N, int64_t K, int r, const float* omega, int l, int iters,
                              __half* L1, __half* L2, __half* R, float* sigma, void* workspace, hipStream_t s) {
  SvdWork w;
  svd_layout(N, K, l, r, &w, static_cast<char*>(workspace));
  hipError_t e;
  // Y = Wt Omega  [N][l]
  if ((e = gemm<__half, float, 0>(Wt, K, 1, omega, l, 1, w.Y, l, nullptr, N, l, K, s)) != hipSuccess) return e;
  if ((e = orthonormalize(w.Y, w.Y2, N, l, w, s)) != hipSuccess) return e;
  for (int it = 0; it < iters; ++it) {
    // Z = Wt^T Y  [K][l]: A(i = k, p = n) = Wt[n K + k]
    if ((e = gemm<__half, float, 0>(Wt, 1, K, w.Y, l, 1, w.Z, l, nullptr, K, l, N, s)) != hipSuccess) return e;
    if ((e = orthonormalize(w.Z, w.Z2, K, l, w, s)) != hipSuccess) return e;
    // Y = Wt Z  [N][l]
    if ((e = gemm<__half, float, 0>(Wt, K, 1, w.Z, l, 1, w.Y, l, nullptr, N, l, K, s)) != hipSuccess) return e;
    if ((e = orthonormalize(w.Y, w.Y2, N, l, w, s)) != hipSuccess) return e;
  }
  // Bm = Y^T Wt  [l][K]: A(i = j, p = n) = Y[n l + j]
  if ((e = gemm<float, __half, 0>(w.Y, 1, l, Wt, K, 1, w.Bm, K, nullptr, l, K, N, s)) != hipSuccess) return e;
  // S = Bm Bm^T (float64), its eigenpairs, the factors' small matrices
  hipLaunchKernelGGL(svd_gram_kernel, dim3((unsigned)((l * l + 255) / 256)), dim3(256), 0, s, w.Bm, (int64_t)1,
                     (int64_t)K, K, l, w.G);
  hipLaunchKernelGGL(svd_eig_kernel, dim3(1), dim3(64), 0, s, w.G, l, r, w.M2, w.M1, sigma ? sigma : w.sigma);
  // L2 = Y M2  [N][r] fp16;  L1 = M1 Bm  [r][K] fp16
  if ((e = gemm<float, float, 1>(w.Y, l, 1, w.M2, r, 1, L2, r, nullptr, N, r, l, s)) != hipSuccess) return e;
  if ((e = gemm<float, float, 1>(w.M1, l, 1, w.Bm, K, 1, L1, K, nullptr, r, K, l, s)) != hipSuccess) return e;
  // R = fp16(Wt - L2 L1)  [N][K]
  return gemm<__half, __half, 2>(L2, r, 1, L1, K, 1, R, K, Wt, N, K, r, s);
}

}  // namespace kq
