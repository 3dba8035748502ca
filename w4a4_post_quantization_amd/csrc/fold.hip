// Offline weight preparation: W' = P^-1 W folded into the weights and quantized along K
// (KroQuant §01: Y = (XP)(P^-1 W); OrbitQuant §03: W' = R^-1 W, R^-1 = R^T), plus the
// column sums wbar = 1^T W used by CentriQ's rank-1 mean restore.  Runs once per
// layer, outside the timed path; written for clarity, one thread per 32-element block.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

#define KQ_INV_SQRT32_F 0.17677669529663688110f

// P^-1 of a 32x32 P into LDS as float: Gauss-Jordan elimination with partial pivoting in
// float64 by the whole workgroup (offline: clarity over speed).  P is either dense
// (row-major, global) or, with ab != NULL, the Kronecker product A (x) B of one block's
// factors ab = {A 4x4, B 8x8} (row-major), formed exactly in float64:
// (A (x) B)[i][j] = A[i/8][j/8] B[i%8][j%8].  A singular P gives non-finite entries.
__device__ void invert32(const float* __restrict__ P, const float* __restrict__ ab, float* __restrict__ pinv) {
  __shared__ double aug[32][64];
  __shared__ double fac[32];
  __shared__ int piv;
  const int t = threadIdx.x, T = blockDim.x;
  for (int e = t; e < 32 * 64; e += T) {
    const int i = e >> 6, j = e & 63;
    if (j >= 32) aug[i][j] = j - 32 == i ? 1.0 : 0.0;
    else if (ab) aug[i][j] = (double)ab[4 * (i >> 3) + (j >> 3)] * (double)ab[16 + 8 * (i & 7) + (j & 7)];
    else aug[i][j] = (double)P[32 * i + j];
  }
  __syncthreads();
  for (int c = 0; c < 32; ++c) {
    if (t == 0) {
      int p = c;
      for (int i = c + 1; i < 32; ++i)
        if (fabs(aug[i][c]) > fabs(aug[p][c])) p = i;
      piv = p;
    }
    __syncthreads();
    if (piv != c && t < 64) {
      const double a = aug[c][t];
      aug[c][t] = aug[piv][t];
      aug[piv][t] = a;
    }
    __syncthreads();
    const double d = aug[c][c];
    __syncthreads();
    if (t < 64) aug[c][t] /= d;
    __syncthreads();
    if (t < 32) fac[t] = t == c ? 0.0 : aug[t][c];
    __syncthreads();
    for (int e = t; e < 32 * 64; e += T) {
      const int i = e >> 6, j = e & 63;
      aug[i][j] -= fac[i] * aug[c][j];
    }
    __syncthreads();
  }
  for (int e = t; e < 32 * 32; e += T) pinv[e] = (float)aug[e >> 5][32 + (e & 31)];
  __syncthreads();
}

// One thread: row n of W^T (= column n of W), block b (32 consecutive k).
// KIND 1: w'_b = (Ai (x) Bi) w_b, i.e. W'm = Ai Wm Bi^T with Wm[k][l] = w_b[8k+l].
// KIND 2: w' = w R (the forward RPBH of the row, since W'^T = W^T R).
// KIND 3: w'_b = P^-1 w_b for a dense block transform P.
// KIND 4: w'_b = (A_b (x) B_b)^-1 w_b with per-block factors (P = AB, float [nb][80]); the
//         grid is 2-D, blockIdx.y = b, so a workgroup inverts one block's P.
// FMT 0: MXFP4 (16 code bytes + 1 E8M0 byte); FMT 2: 2-bit Lloyd-Max + fp16 group scale.
// W element (n, k) sits at n * sn + k * sk: sn = K, sk = 1 for [N][K] weights, sn = 1,
// sk = N for [K][N].  With [K][N] weights consecutive threads take consecutive n (the
// reads of a warp then cover contiguous memory).
template <int KIND, int FMT>
__global__ __launch_bounds__(256) void fold_kernel(const __half* __restrict__ W, int64_t N, int64_t K, int64_t sn,
                                                   int64_t sk, KronFactors fi,
                                                   const int32_t* __restrict__ perm, const int8_t* __restrict__ sign,
                                                   const float* __restrict__ P, const int8_t* __restrict__ pts,
                                                   float t4, uint8_t* __restrict__ wcodes, void* __restrict__ wscales) {
  __shared__ float pinv[KIND >= 3 ? 32 * 32 : 1];
  if (KIND == 3) invert32(P, nullptr, pinv);          // every thread of the workgroup takes part
  if (KIND == 4) invert32(nullptr, P + (int64_t)blockIdx.y * 80, pinv);
  const int64_t nb = K >> 5;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (KIND == 4 ? id >= N : id >= N * nb) return;
  const bool nfast = sn == 1;
  const int64_t n = KIND == 4 ? id : (nfast ? id % N : id / nb);
  const int64_t b = KIND == 4 ? (int64_t)blockIdx.y : (nfast ? id / N : id % nb);
  const __half* wr = W + n * sn;
  float w[32], y[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t k = 32 * b + i;
    const int64_t src = KIND == 2 ? (int64_t)perm[k] : k;
    w[i] = __half2float(wr[src * sk]);
    if (pts) w[i] = ldexpf(w[i], (int)pts[src]);   // W' = P^-1 D W with D = diag(2^pts), exact
  }
  if (KIND == 1) {
    float z[32];  // Z = Wm Bi^T : Z[k][j] = sum_l Wm[k][l] Bi[j][l]
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int l = 0; l < 8; ++l) acc = __builtin_fmaf(w[8 * k + l], fi.B[8 * j + l], acc);
        z[8 * k + j] = acc;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(fi.A[4 * i + k], z[8 * k + j], acc);
        y[8 * i + j] = acc;
      }
  } else if (KIND >= 3) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) acc = __builtin_fmaf(pinv[32 * i + j], w[j], acc);
      y[i] = acc;
    }
  } else if (KIND == 2) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (!(i & h)) { const float a = w[i], c = w[i + h]; w[i] = a + c; w[i + h] = a - c; }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float d = sign[32 * b + i] < 0 ? -KQ_INV_SQRT32_F : KQ_INV_SQRT32_F;
      y[i] = __builtin_fmaf(w[i], d, 0.0f);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = w[i] + 0.0f;
  }

  if (FMT == 0) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(y[i]));
    const uint32_t sb = e8m0_byte(a);
    const float sc = e8m0_as_cvt_scale(sb);
    uint4 out;
    out.x = cvt8_fp4(y + 0, sc);
    out.y = cvt8_fp4(y + 8, sc);
    out.z = cvt8_fp4(y + 16, sc);
    out.w = cvt8_fp4(y + 24, sc);
    reinterpret_cast<uint4*>(wcodes + n * (K >> 1))[b] = out;
    reinterpret_cast<uint8_t*>(wscales)[n * nb + b] = (uint8_t)sb;
  } else {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ss = __builtin_fmaf(y[i], y[i], ss);
    const __half sh = __float2half_rn(sqrtf(ss / 32.0f));
    const float s = __half2float(sh);
    const float thr = t4 * s;
    uint32_t lo = 0, hi = 0;
    if (s > 0.0f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t c = (fabsf(y[i]) > thr ? 1u : 0u) | (y[i] < 0.0f ? 2u : 0u);
        if (i < 16) lo |= c << (2 * i);
        else hi |= c << (2 * (i - 16));
      }
    }
    reinterpret_cast<uint2*>(wcodes + n * (K >> 2))[b] = make_uint2(lo, hi);
    reinterpret_cast<__half*>(wscales)[n * nb + b] = sh;
  }
}

// wbar[n] = fp16(sum_k W(n, k)), summed in float64 (one rounding at the end, so wbar is
// the fp16 rounding of the column sum up to float64 summation error).  The conversion is
// LLVM's direct f64 -> f16 truncation, a single round-to-nearest-even.
__device__ __forceinline__ __half f64_to_f16(double v) {
  return __builtin_bit_cast(__half, (_Float16)v);
}
// [N][K] weights: one wavefront per n, lanes striding over k, then a wavefront sum.
__global__ __launch_bounds__(256) void colsum_kernel(const __half* __restrict__ W, int64_t N, int64_t K,
                                                     __half* __restrict__ wbar) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  double acc = 0.0;
  for (int64_t k = lane; k < K; k += 64) acc += (double)__half2float(W[n * K + k]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) wbar[n] = f64_to_f16(acc);
}

// [K][N] weights: one thread per n walking down its column (a warp reads contiguous rows).
__global__ __launch_bounds__(256) void colsum_kn_kernel(const __half* __restrict__ W, int64_t N, int64_t K,
                                                        __half* __restrict__ wbar) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) acc += (double)__half2float(W[k * N + n]);
  wbar[n] = f64_to_f16(acc);
}

template <int KIND>
static void fold_fmt(int fmt, dim3 g, dim3 b, hipStream_t s, const __half* W, int64_t N, int64_t K, int64_t sn,
                     int64_t sk, const KronFactors& fi, const int32_t* perm, const int8_t* sign, const float* P,
                     const int8_t* pts, float t4, uint8_t* wc, void* ws) {
  if (fmt == 0)
    hipLaunchKernelGGL((fold_kernel<KIND, 0>), g, b, 0, s, W, N, K, sn, sk, fi, perm, sign, P, pts, t4, wc, ws);
  else
    hipLaunchKernelGGL((fold_kernel<KIND, 2>), g, b, 0, s, W, N, K, sn, sk, fi, perm, sign, P, pts, t4, wc, ws);
}

hipError_t launch_fold(int kind, int fmt, bool kn, const __half* W, int64_t N, int64_t K, const KronFactors& finv,
                       const int32_t* perm, const int8_t* sign, const float* P, const int8_t* pts, uint8_t* wcodes,
                       void* wscales, hipStream_t s) {
  const int64_t total = N * (K / 32);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  const float t4 = lm_tables().t4;
  const int64_t sn = kn ? 1 : K, sk = kn ? N : 1;
  if (kind == 4) {
    const dim3 g2((unsigned)((N + 255) / 256), (unsigned)(K / 32));
    fold_fmt<4>(fmt, g2, block, s, W, N, K, sn, sk, finv, perm, sign, P, pts, t4, wcodes, wscales);
  } else if (kind == 1) {
    fold_fmt<1>(fmt, grid, block, s, W, N, K, sn, sk, finv, perm, sign, P, pts, t4, wcodes, wscales);
  } else if (kind == 2) {
    fold_fmt<2>(fmt, grid, block, s, W, N, K, sn, sk, finv, perm, sign, P, pts, t4, wcodes, wscales);
  } else if (kind == 3) {
    fold_fmt<3>(fmt, grid, block, s, W, N, K, sn, sk, finv, perm, sign, P, pts, t4, wcodes, wscales);
  } else {
    fold_fmt<0>(fmt, grid, block, s, W, N, K, sn, sk, finv, perm, sign, P, pts, t4, wcodes, wscales);
  }
  return hipGetLastError();
}

hipError_t launch_colsum(bool kn, const __half* W, int64_t N, int64_t K, __half* wbar, hipStream_t s) {
  if (kn)
    hipLaunchKernelGGL(colsum_kn_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, W, N, K, wbar);
  else
    hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, W, N, K, wbar);
  return hipGetLastError();
}

}  // namespace kq
