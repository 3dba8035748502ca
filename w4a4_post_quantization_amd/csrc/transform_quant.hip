// Online activation path: [centre] -> 32-element block transform -> 4-bit quantize+pack.
//
// KroQuant (§02): each 32-element block x_b becomes x_b (A (x) B).  With the block seen
// as a 4x8 matrix Xm[i][j] = x_b[8i+j] this is Ym = A^T Xm B: one lane of a quad holds
// one row of Xm (8 fp16 = 16 contiguous bytes), multiplies it by B in registers, and the
// quad mixes its four rows by A^T with DPP quad broadcasts.
// OrbitQuant (§03): RPBH = x . Pi . blockdiag(H32) . D / sqrt(32); the row is staged in
// LDS for the full-K permutation gather, each lane then runs three in-register Hadamard
// butterfly stages and two cross-lane (DPP) stages.
// CentriQ (arXiv abstract): the token mean is subtracted before the rotation and stored
// as fp16 for the rank-1 restore in the linear.
// MXFP4 (KroQuant §03, OCP MX v1.0): per block the E8M0 exponent of max|y| and
// round-to-nearest-even E2M1 codes, converted and packed in the same pass with the
// gfx950 scaled FP4 conversion.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

// 1/sqrt(32) rounded to float.
#define KQ_INV_SQRT32 0.17677669529663688110f

// Ym row `qi` of one Kronecker block: this lane holds Xm[qi][:] in x, acol[i] = A[i][qi].
// Every accumulation starts from +0, so an exact zero result is +0, never -0.
__device__ __forceinline__ void kron_quad(const float* x, const KronFactors& f, const float* acol, float* y) {
  float z[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_fmaf(x[j], f.B[8 * j + l], acc);
    z[l] = acc;
  }
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    float acc = 0.0f;
    acc = __builtin_fmaf(acol[0], quad_bcast<0>(z[l]), acc);
    acc = __builtin_fmaf(acol[1], quad_bcast<1>(z[l]), acc);
    acc = __builtin_fmaf(acol[2], quad_bcast<2>(z[l]), acc);
    acc = __builtin_fmaf(acol[3], quad_bcast<3>(z[l]), acc);
    y[l] = acc;
  }
}

__device__ __forceinline__ void kron_acol(const KronFactors& f, int qi, float* acol) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = f.A[4 * i + 0];
    a = qi == 1 ? f.A[4 * i + 1] : a;
    a = qi == 2 ? f.A[4 * i + 2] : a;
    a = qi == 3 ? f.A[4 * i + 3] : a;
    acol[i] = a;
  }
}

// Sylvester Hadamard over the 32 elements held by a quad (8 per lane, element 8*qi+m).
// Index bits 0-2 are in-lane butterflies; bits 3-4 pair lanes qi^1 and qi^2.  A lane
// whose quad index has bit b set computes own - partner (the negated butterfly output),
// so the result equals (-1)^popcount(qi) times the true transform; callers fold that
// sign into the per-element output coefficient.
__device__ __forceinline__ void hadamard32_quad(float* v, float s1, float s2) {
#pragma unroll
  for (int m = 0; m < 8; m += 2) { float a = v[m], b = v[m + 1]; v[m] = a + b; v[m + 1] = a - b; }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m & 2) continue;
    float a = v[m], b = v[m + 2]; v[m] = a + b; v[m + 2] = a - b;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) { float a = v[m], b = v[m + 4]; v[m] = a + b; v[m + 4] = a - b; }
#pragma unroll
  for (int m = 0; m < 8; ++m) v[m] = __builtin_fmaf(quad_xor1(v[m]), s1, v[m]);
#pragma unroll
  for (int m = 0; m < 8; ++m) v[m] = __builtin_fmaf(quad_xor2(v[m]), s2, v[m]);
}

// ---------------------------------------------------------------------------------
// Streaming Kronecker + MXFP4: the activations are a flat sequence of 32-element blocks
// (rows are contiguous and K % 32 == 0).  A wavefront handles 16 blocks (1 KiB of input,
// one 16-byte load per lane, fully coalesced) per step and writes 256 contiguous bytes
// of codes and 16 scale bytes.
template <int U>
__global__ __launch_bounds__(256) void kron_mx_stream_kernel(const uint4* __restrict__ X, int64_t nblocks,
                                                             KronFactors f, uint32_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int qi = lane & 3;
  float acol[4];
  kron_acol(f, qi, acol);
  const int64_t nchunks = (nblocks + 15) >> 4;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  for (int64_t c0 = wave; c0 < nchunks; c0 += nwaves * U) {
    uint4 raw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * nwaves;
      ok[u] = (c < nchunks) && (c * 16 + (lane >> 2) < nblocks);
      raw[u] = ok[u] ? X[c * 64 + lane] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[8], y[8];
      unpack8_f16(raw[u], x);
      kron_quad(x, f, acol, y);
      float m = 0.0f;
#pragma unroll
      for (int l = 0; l < 8; ++l) m = fmaxf(m, fabsf(y[l]));
      m = quad_max(m);
      const uint32_t sb = e8m0_byte(m);
      const uint32_t w = cvt8_fp4(y, e8m0_as_cvt_scale(sb));
      const int64_t c = c0 + u * nwaves;
      if (ok[u]) {
        codes[c * 64 + lane] = w;
        if (qi == 0) scales[c * 16 + (lane >> 2)] = (uint8_t)sb;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Row-staged kernel: one workgroup per token row (grid-strided).  Thread t owns the
// 8-element groups g = t + T*j (j < NG); a group's quad holds one 32-element block.
// KIND: 0 none, 1 Kronecker, 2 RPBH.  FMT: 0 MXFP4, 1 per-token Lloyd-Max (LM4).
template <int KIND, int FMT, bool CENTER, int NG>
__global__ __launch_bounds__(1024) void row_quant_kernel(const __half* __restrict__ X, int64_t M, int K,
                                                         KronFactors f, const int32_t* __restrict__ perm,
                                                         const int8_t* __restrict__ sign, LmTables lm,
                                                         uint8_t* __restrict__ codes, void* __restrict__ scales,
                                                         __half* __restrict__ mu) {
  extern __shared__ __align__(16) unsigned char smem[];
  __half* srow = reinterpret_cast<__half*>(smem);
  float* red = reinterpret_cast<float*>(smem + (KIND == 2 ? (size_t)K * 2 : 0));
  const int t = threadIdx.x, T = blockDim.x, lane = t & 63, wid = t >> 6, nw = T >> 6;
  const int G = K >> 3;
  const int qi = lane & 3;

  float acol[4];
  if (KIND == 1) kron_acol(f, qi, acol);
  // RPBH: gather indices and output coefficients d_j * (-1)^popcount(qi) / sqrt(32)
  uint32_t pidx[KIND == 2 ? NG : 1][4];
  float coef[KIND == 2 ? NG : 1][8];
  const float s1 = (qi & 1) ? -1.0f : 1.0f;
  const float s2 = (qi & 2) ? -1.0f : 1.0f;
  if (KIND == 2) {
    const float rho = s1 * s2 * KQ_INV_SQRT32;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = t + T * j;
      const bool v = g < G;
#pragma unroll
      for (int m = 0; m < 8; m += 2) {
        const uint32_t p0 = v ? (uint32_t)perm[8 * g + m] : 0u;
        const uint32_t p1 = v ? (uint32_t)perm[8 * g + m + 1] : 0u;
        pidx[j][m >> 1] = p0 | (p1 << 16);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) coef[j][m] = (v && sign[8 * g + m] < 0) ? -rho : rho;
    }
  }

  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    const uint4* xr = reinterpret_cast<const uint4*>(X + row * (int64_t)K);
    uint4 raw[NG];
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = t + T * j;
      raw[j] = g < G ? xr[g] : make_uint4(0u, 0u, 0u, 0u);
      if (KIND == 2 && g < G) reinterpret_cast<uint4*>(srow)[g] = raw[j];
      if (CENTER) {
        float x[8];
        unpack8_f16(raw[j], x);
#pragma unroll
        for (int m = 0; m < 8; ++m) psum += x[m];
      }
    }
    float muf = 0.0f;
    if (CENTER) {
      const float s = wave_sum(psum);
      if (lane == 0) red[wid] = s;
      __syncthreads();
      float tot = 0.0f;
      for (int w = 0; w < nw; ++w) tot += red[w];
      const __half mh = __float2half_rn(tot / (float)K);
      muf = __half2float(mh);
      if (t == 0) mu[row] = mh;
    } else if (KIND == 2) {
      __syncthreads();
    }

    float yv[FMT == 1 ? NG : 1][8];
    float ssq = 0.0f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = t + T * j;
      const bool valid = g < G;
      float u[8], y[8];
      if (KIND == 2) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t p = (pidx[j][m >> 1] >> (16 * (m & 1))) & 0xFFFFu;
          u[m] = __half2float(srow[p]);
        }
      } else {
        unpack8_f16(raw[j], u);
      }
      if (CENTER) {
#pragma unroll
        for (int m = 0; m < 8; ++m) u[m] = u[m] - muf;
      }
      if (KIND == 1) {
        kron_quad(u, f, acol, y);
      } else if (KIND == 2) {
        hadamard32_quad(u, s1, s2);
#pragma unroll
        for (int m = 0; m < 8; ++m) y[m] = __builtin_fmaf(u[m], coef[j][m], 0.0f);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) y[m] = u[m] + 0.0f;
      }
      if (FMT == 0) {
        float a = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) a = fmaxf(a, fabsf(y[m]));
        a = quad_max(a);
        const uint32_t sb = e8m0_byte(a);
        const uint32_t w = cvt8_fp4(y, e8m0_as_cvt_scale(sb));
        if (valid) {
          reinterpret_cast<uint32_t*>(codes + row * (int64_t)(K >> 1))[g] = w;
          if (qi == 0) reinterpret_cast<uint8_t*>(scales)[row * (int64_t)(K >> 5) + (g >> 2)] = (uint8_t)sb;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          yv[j][m] = y[m];
          // lanes past the end of the row (K/8 not a multiple of the block size) hold
          // gathered filler and must not enter the token's sum of squares
          ssq = valid ? __builtin_fmaf(y[m], y[m], ssq) : ssq;
        }
      }
    }

    if (FMT == 1) {
      const float s = wave_sum(ssq);
      if (lane == 0) red[32 + wid] = s;
      __syncthreads();
      float tot = 0.0f;
      for (int w = 0; w < nw; ++w) tot += red[32 + w];
      const float sc = sqrtf(tot / (float)K);
      float ts[7];
#pragma unroll
      for (int i = 0; i < 7; ++i) ts[i] = lm.t16[i] * sc;
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const int g = t + T * j;
        uint32_t w = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          // number of thresholds strictly below |y| (a value on a threshold takes the
          // smaller magnitude), by a three-step binary search
          const float a = fabsf(yv[j][m]);
          uint32_t idx = a > ts[3] ? 4u : 0u;
          const float t1 = idx ? ts[5] : ts[1];
          idx += a > t1 ? 2u : 0u;
          const float t0 = idx == 0 ? ts[0] : idx == 2 ? ts[2] : idx == 4 ? ts[4] : ts[6];
          idx += a > t0 ? 1u : 0u;
          const uint32_t code = idx | (yv[j][m] < 0.0f ? 8u : 0u);
          w |= code << (4 * m);
        }
        if (g < G) reinterpret_cast<uint32_t*>(codes + row * (int64_t)(K >> 1))[g] = w;
      }
      if (t == 0) reinterpret_cast<float*>(scales)[row] = sc;
    }
    __syncthreads();
  }
}

int device_cu_count() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
  }();
  return cus;
}

hipError_t launch_kron_mx_stream(const __half* X, int64_t nblocks, const KronFactors& f, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  constexpr int U = 2;
  const int64_t nchunks = (nblocks + 15) / 16;
  const int64_t waves = (nchunks + U - 1) / U;
  int64_t grid = (waves + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kron_mx_stream_kernel<U>, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(X), nblocks, f, reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

template <int KIND, int FMT, bool CENTER>
static hipError_t row_launch_ng(int ng, unsigned grid, unsigned threads, size_t lds, const __half* X, int64_t M,
                                int K, const KronFactors& f, const int32_t* perm, const int8_t* sign,
                                uint8_t* codes, void* scales, __half* mu, hipStream_t s) {
  const LmTables& lm = lm_tables();
  switch (ng) {
    case 1: hipLaunchKernelGGL((row_quant_kernel<KIND, FMT, CENTER, 1>), dim3(grid), dim3(threads), lds, s, X, M, K, f, perm, sign, lm, codes, scales, mu); break;
    case 2: hipLaunchKernelGGL((row_quant_kernel<KIND, FMT, CENTER, 2>), dim3(grid), dim3(threads), lds, s, X, M, K, f, perm, sign, lm, codes, scales, mu); break;
    case 3: hipLaunchKernelGGL((row_quant_kernel<KIND, FMT, CENTER, 3>), dim3(grid), dim3(threads), lds, s, X, M, K, f, perm, sign, lm, codes, scales, mu); break;
    default: hipLaunchKernelGGL((row_quant_kernel<KIND, FMT, CENTER, 4>), dim3(grid), dim3(threads), lds, s, X, M, K, f, perm, sign, lm, codes, scales, mu); break;
  }
  return hipGetLastError();
}

template <int KIND>
static hipError_t row_launch_kind(int fmt, bool center, int ng, unsigned grid, unsigned threads, size_t lds,
                                  const __half* X, int64_t M, int K, const KronFactors& f, const int32_t* perm,
                                  const int8_t* sign, uint8_t* codes, void* scales, __half* mu, hipStream_t s) {
  if (fmt == 0) {
    return center ? row_launch_ng<KIND, 0, true>(ng, grid, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s)
                  : row_launch_ng<KIND, 0, false>(ng, grid, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
  }
  return center ? row_launch_ng<KIND, 1, true>(ng, grid, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s)
                : row_launch_ng<KIND, 1, false>(ng, grid, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
}

hipError_t launch_row_quant(int kind, int fmt, bool center, const __half* X, int64_t M, int64_t K,
                            const KronFactors& f, const int32_t* perm, const int8_t* sign, uint8_t* codes,
                            void* scales, __half* mu, hipStream_t s) {
  const int G = (int)(K / 8);
  int threads = ((G + 63) / 64) * 64;
  if (threads > 1024) threads = 1024;
  const int ng = (G + threads - 1) / threads;       // <= 4 for K <= 32768
  const size_t lds = (kind == 2 ? (size_t)K * 2 : 0) + 64 * sizeof(float);
  int64_t grid = M;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  switch (kind) {
    case 1: return row_launch_kind<1>(fmt, center, ng, (unsigned)grid, threads, lds, X, M, (int)K, f, perm, sign, codes, scales, mu, s);
    case 2: return row_launch_kind<2>(fmt, center, ng, (unsigned)grid, threads, lds, X, M, (int)K, f, perm, sign, codes, scales, mu, s);
    default: return row_launch_kind<0>(fmt, center, ng, (unsigned)grid, threads, lds, X, M, (int)K, f, perm, sign, codes, scales, mu, s);
  }
}

}  // namespace kq
