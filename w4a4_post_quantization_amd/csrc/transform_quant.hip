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

#include <map>
#include <mutex>
#include <tuple>

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
// Row-staged kernel: each workgroup walks token rows (grid-strided).  Thread t owns the
// 8-element groups g = t + T*j (j < NG) of a row; a group's quad holds one 32-element
// block.  The next row's 16-byte chunks are loaded into registers while the current row
// is transformed, and rows alternate between two LDS buffers, so one barrier per row
// suffices and two rows per workgroup are in flight.
// KIND: 0 none, 1 Kronecker, 2 RPBH.  FMT: 0 MXFP4, 1 per-token Lloyd-Max (LM4).
template <int KIND, int FMT, bool CENTER, int NG>
__global__ __launch_bounds__(512) void row_quant_kernel(const __half* __restrict__ X, int64_t M, int K,
                                                        KronFactors f, const int32_t* __restrict__ perm,
                                                        const int8_t* __restrict__ sign, LmTables lm,
                                                        uint8_t* __restrict__ codes, void* __restrict__ scales,
                                                        __half* __restrict__ mu) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int t = threadIdx.x, T = blockDim.x, lane = t & 63, wid = t >> 6, nw = T >> 6;
  const int G = K >> 3;
  const int qi = lane & 3;
  // two row buffers of K halves (RPBH only), addressed from the __shared__ base so the
  // gathers stay LDS reads
  __half* const srow0 = reinterpret_cast<__half*>(smem);
  float* red = reinterpret_cast<float*>(smem + (KIND == 2 ? (size_t)K * 4 : 0));   // [2][32]: wave sums

  float acol[4];
  if (KIND == 1) kron_acol(f, qi, acol);
  // RPBH: gather indices (K <= 16384 uses 14 bits; bit 15 carries the sign d_j of the
  // output element), and the lane's butterfly sign (-1)^popcount(qi) folded into 1/sqrt(32)
  uint32_t pidx[KIND == 2 ? NG : 1][4];
  const float s1 = (qi & 1) ? -1.0f : 1.0f;
  const float s2 = (qi & 2) ? -1.0f : 1.0f;
  const float rho = s1 * s2 * KQ_INV_SQRT32;
  if (KIND == 2) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = t + T * j;
      const bool v = g < G;
#pragma unroll
      for (int m = 0; m < 8; m += 2) {
        uint32_t p0 = 0, p1 = 0;
        if (v) {
          p0 = (uint32_t)perm[8 * g + m] | (sign[8 * g + m] < 0 ? 0x8000u : 0u);
          p1 = (uint32_t)perm[8 * g + m + 1] | (sign[8 * g + m + 1] < 0 ? 0x8000u : 0u);
        }
        pidx[j][m >> 1] = p0 | (p1 << 16);
      }
    }
  }

  uint4 raw[NG];
  auto load_row = [&](int64_t row) {
    const uint4* xr = reinterpret_cast<const uint4*>(X + row * (int64_t)K);
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = t + T * j;
      raw[j] = (row < M && g < G) ? xr[g] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  int64_t row = blockIdx.x;
  load_row(row);
  for (int it = 0; row < M; row += gridDim.x, ++it) {
    const int buf = it & 1;
    uint4 cur[NG];
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      cur[j] = raw[j];
      const int g = t + T * j;
      if (KIND == 2 && g < G) reinterpret_cast<uint4*>(srow0 + buf * K)[g] = cur[j];
      if (CENTER) {
        float x[8];
        unpack8_f16(cur[j], x);
#pragma unroll
        for (int m = 0; m < 8; ++m) psum += x[m];
      }
    }
    load_row(row + gridDim.x);            // prefetch the next row while this one is processed
    float* rd = red + buf * 32;
    if (CENTER) {
      const float sw = wave_sum(psum);
      if (lane == 0) rd[wid] = sw;
    }
    if (CENTER || KIND == 2) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    float muf = 0.0f;
    if (CENTER) {
      float tot = 0.0f;
      for (int w = 0; w < nw; ++w) tot += rd[w];
      const __half mh = __float2half_rn(tot / (float)K);
      muf = __half2float(mh);
      if (t == 0) mu[row] = mh;
    }

    float yv[FMT == 1 ? NG : 1][8];
    float ssq = 0.0f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int g = t + T * j;
      const bool valid = g < G;
      float u[8], y[8];
      uint32_t sgn = 0;
      if (KIND == 2) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t p = (pidx[j][m >> 1] >> (16 * (m & 1))) & 0xFFFFu;
          u[m] = __half2float(srow0[buf * K + (int)(p & 0x7FFFu)]);
          sgn |= (p >> 15) << m;
        }
      } else {
        unpack8_f16(cur[j], u);
      }
      if (CENTER) {
#pragma unroll
        for (int m = 0; m < 8; ++m) u[m] = u[m] - muf;
      }
      if (KIND == 1) {
        kron_quad(u, f, acol, y);
      } else if (KIND == 2) {
        hadamard32_quad(u, s1, s2);
        // y = v d_j / sqrt(32); the fma with +0 turns an exact -0 into +0
#pragma unroll
        for (int m = 0; m < 8; ++m) y[m] = __builtin_fmaf(u[m], ((sgn >> m) & 1) ? -rho : rho, 0.0f);
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
          // lanes past the end of the row hold gathered filler and must not enter the
          // token's sum of squares
          ssq = valid ? __builtin_fmaf(y[m], y[m], ssq) : ssq;
        }
      }
    }

    if (FMT == 1) {
      const float sw = wave_sum(ssq);
      if (lane == 0) rd[16 + wid] = sw;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      float tot = 0.0f;
      for (int w = 0; w < nw; ++w) tot += rd[16 + w];
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
  }
}

// ---------------------------------------------------------------------------------
// Matrix-core block transform.  A 32-element block transform is a 32x32 matrix product,
// so 16 blocks at a time go through v_mfma_f32_16x16x32_f16 in the transposed
// orientation C^T = P^T X^T: the A operand holds 16 output rows of P^T (two 16-row
// tiles cover the block), the B operand holds the 16 blocks as columns (lane l: block
// l%16, elements 8(l/16)..+7 as fp16, exact), and lane l ends with outputs
// 4q..4q+3 and 16+4q..16+4q+3 (q = l/16) of block l%16 -- eight outputs of one block
// per lane, so the block maximum needs two lane exchanges and the codes pack locally.
// RPBH: P = H32, entries +-1, exact in fp16.  Kronecker: P = A (x) B formed in float32
// and split into fp16 hi + lo parts (two MFMAs per tile; the split keeps ~22 bits).

struct MfmaXform {
  v8h a[2][2];   // [tile][hi, lo] A-operand fragments (P^T rows)
};

// A-operand fragments of P^T for this lane: tile t rows j = 16t + l%16, k = 8q..8q+7.
__device__ __forceinline__ MfmaXform mfma_xform_kron(const KronFactors& f, int lane) {
  MfmaXform x;
  const int q = lane >> 4, jl = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * t + jl;                 // output index (column of P)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * q + i;                 // input index (row of P)
      const float p = f.A[4 * (k >> 3) + (j >> 3)] * f.B[8 * (k & 7) + (j & 7)];
      const _Float16 hi = (_Float16)p;
      x.a[t][0][i] = hi;
      x.a[t][1][i] = (_Float16)(p - (float)hi);
    }
  }
  return x;
}

__device__ __forceinline__ MfmaXform mfma_xform_hadamard(int lane) {
  MfmaXform x;
  const int q = lane >> 4, jl = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * t + jl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * q + i;
      x.a[t][0][i] = (__builtin_popcount(j & k) & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
      x.a[t][1][i] = (_Float16)0.0f;
    }
  }
  return x;
}

// y[0..3] = outputs 4q..4q+3, y[4..7] = outputs 16+4q..16+4q+3 of block l%16.
template <bool LO>
__device__ __forceinline__ void mfma_block_transform(const MfmaXform& x, const v8h& b, float* y) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(x.a[t][0], b, acc, 0, 0, 0);
    if (LO) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(x.a[t][1], b, acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[4 * t + i] = acc[i];
  }
}

// MXFP4 of the lane's eight outputs: block maximum over the four lanes l, l^16, l^32,
// l^48, E8M0 byte, and the packed codes as one dword per lane at byte offset
// {0, 8, 4, 12}[q] of the block's 16 code bytes (lanes q and q^1 swap halves).
// Inputs must not be -0.0.
__device__ __forceinline__ void mx_pack_block(const float* y, int q, uint32_t& dword, int& byte_off,
                                              uint32_t& scale_byte) {
  float a = fmaxf(fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))),
                  fmaxf(fmaxf(fabsf(y[4]), fabsf(y[5])), fmaxf(fabsf(y[6]), fabsf(y[7]))));
  // maximum with lanes l^16 and l^32 through the register lane swaps: each swap returns,
  // per lane, its own value in one result and its partner's in the other, so the maximum
  // of both results is the pairwise maximum whichever way round the swap goes
  {
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = fmaxf(a, fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1])));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = fmaxf(a, fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1])));
  }
  const uint32_t sb = e8m0_byte(a);
  const float sc = e8m0_as_cvt_scale(sb);
  uint32_t h0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], sc, 0);
  h0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h0, y[2], y[3], sc, 1);      // bytes 2q, 2q+1
  uint32_t h1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[4], y[5], sc, 0);
  h1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h1, y[6], y[7], sc, 1);      // bytes 8+2q, 8+2q+1
  // lanes of an even row (q even) keep h0 and receive the odd partner's h0; lanes of an
  // odd row receive the even partner's h1 and keep h1 -- one row swap of the two registers
  // (the odd rows of the first with the even rows of the second)
  const auto sw = __builtin_amdgcn_permlane16_swap(h0, h1, false, false);
  dword = sw[0] | (sw[1] << 16);
  byte_off = (q & 1) ? 8 + 2 * (q - 1) : 2 * q;
  scale_byte = sb;
}

// Streaming Kronecker (or identity) + MXFP4 on the matrix cores: the activations are a
// flat sequence of 32-element blocks; a wavefront handles 16 blocks (1 KiB) per step with
// one 16-byte load per lane and writes 256 contiguous code bytes.
template <int U, bool KRON>
__global__ __launch_bounds__(256) void kron_mx_mfma_stream_kernel(const uint4* __restrict__ X, int64_t nblocks,
                                                                  KronFactors f, uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, q = lane >> 4, bl = lane & 15;
  MfmaXform xf;
  if (KRON) {
    xf = mfma_xform_kron(f, lane);
  } else {   // identity: P^T rows are unit vectors
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xf.a[t][0][i] = (16 * t + bl == 8 * q + i) ? (_Float16)1.0f : (_Float16)0.0f;
        xf.a[t][1][i] = (_Float16)0.0f;
      }
  }
  const int64_t nchunks = (nblocks + 15) >> 4;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  for (int64_t c0 = wave; c0 < nchunks; c0 += nwaves * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * nwaves;
      const int64_t blk = c * 16 + bl;
      raw[u] = (c < nchunks && blk < nblocks) ? X[blk * 4 + q] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[8];
      mfma_block_transform<KRON>(xf, __builtin_bit_cast(v8h, raw[u]), y);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] += 0.0f;      // an exact zero leaves as +0
      uint32_t w, sb;
      int off;
      mx_pack_block(y, q, w, off, sb);
      const int64_t c = c0 + u * nwaves;
      const int64_t blk = c * 16 + bl;
      if (c < nchunks && blk < nblocks) {
        *reinterpret_cast<uint32_t*>(codes + blk * 16 + off) = w;
        if (q == 0) scales[blk] = (uint8_t)sb;
      }
    }
  }
}

// Row-staged RPBH + MXFP4 on the matrix cores, optional centring.  Workgroups are
// persistent (one launch fills the chip once) and build, once, an LDS gather table of
// the permutation (u16 per element) and a sign bitmask per block, so the per-row work
// is only the row itself.  WPR wavefronts share a row (NR = 8 / WPR rows in flight per
// workgroup, each in its own LDS slot); with WPR = 1 every wavefront owns its rows and
// needs no workgroup barrier.  A wavefront loads its share of the next row into
// registers while it transforms the current one.
// Centring is applied after the rotation: (x - mu 1) H32 = x H32 - 32 mu e_0 for the
// Sylvester matrix (every column but the first sums to zero), so only output 0 of each
// block is corrected; the result is the same linear map as centring first.
constexpr int RPBH_WAVES = 8;
constexpr int RPBH_LMAX = 6;   // 16-byte row chunks per lane per row, at most

__host__ __device__ constexpr size_t rpbh_lds_bytes(int wpr, int K) {
  return (size_t)(RPBH_WAVES / wpr) * K * 2 + (size_t)K * 2 + (size_t)(K / 32) * 4 + RPBH_WAVES * 4;
}

struct RowChunks {
  v4u v[RPBH_LMAX];
};

// The lane's 16-byte chunks cidx[] of row `row` (rows past M read row M-1).
__device__ __forceinline__ RowChunks rpbh_load_row(const __half* __restrict__ X, int64_t row, int64_t M, int K,
                                                   const int* cidx) {
  const v4u* xr = reinterpret_cast<const v4u*>(X + (row < M ? row : M - 1) * (int64_t)K);
  RowChunks r;
#pragma unroll
  for (int j = 0; j < RPBH_LMAX; ++j) r.v[j] = xr[cidx[j]];
  return r;
}

template <bool CENTER, int WPR>
__global__ __launch_bounds__(64 * RPBH_WAVES) void rpbh_mx_mfma_rows_kernel(
    const __half* __restrict__ X, int64_t M, int K, const int32_t* __restrict__ perm,
    const int8_t* __restrict__ sign, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    __half* __restrict__ mu) {
  constexpr int NR = RPBH_WAVES / WPR;
  extern __shared__ __align__(16) unsigned char smem[];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int rs = wid / WPR, wr = wid % WPR;   // row slot of this wave, its index within the row
  const int q = lane >> 4, bl = lane & 15;
  const int G = K >> 3, nb = K >> 5, nchunk = (nb + 15) >> 4;
  __half* const rows = reinterpret_cast<__half*>(smem);                                        // [NR][K]
  uint16_t* const tab = reinterpret_cast<uint16_t*>(smem + (size_t)NR * K * 2);               // [K]
  uint32_t* const smask = reinterpret_cast<uint32_t*>(smem + (size_t)NR * K * 2 + (size_t)K * 2);   // [nb]
  float* const red = reinterpret_cast<float*>(smask + nb);                                    // [8]

  __half* const slot = rows + (size_t)rs * K;
  const int nl = (G + 64 * WPR - 1) / (64 * WPR);
  // Loads and LDS writes use clamped indices instead of conditions (a lane past the end
  // repeats the last chunk, rows past M repeat row M-1, chunks j >= nl -- only when
  // K < 3072 WPR -- repeat chunk nl - 1, and the duplicate writes carry identical data),
  // so no load is placed in a branch together with its consumer.
  int cidx[RPBH_LMAX];
#pragma unroll
  for (int j = 0; j < RPBH_LMAX; ++j) {
    const int c = wr * 64 + lane + 64 * WPR * (j < nl ? j : nl - 1);
    cidx[j] = c < G ? c : G - 1;
  }
  RowChunks raw;
  const int64_t stride = (int64_t)gridDim.x * NR;
  int64_t base = (int64_t)blockIdx.x * NR;

  // gather table (u16 per element) and sign masks (bit j of smask[b]: d_{32b+j} < 0).
  // Every load of the set-up and of the first row is issued before any is waited for.
  // 16-byte perm chunks per thread: K <= 3072 WPR (so that G <= 384 WPR) and K <= 16384
  constexpr int PV = WPR == 1 ? 2 : WPR == 2 ? 3 : WPR == 4 ? 6 : 8;
  uint4 pv[PV];
#pragma unroll
  for (int i = 0; i < PV; ++i) {
    const int c = min(t + 64 * RPBH_WAVES * i, (K >> 2) - 1);
    pv[i] = reinterpret_cast<const uint4*>(perm)[c];
  }
  const int sb_ = min(t, nb - 1);                      // this thread's block of sign bytes (nb <= 512)
  uint32_t sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = reinterpret_cast<const uint32_t*>(sign + 32 * sb_)[i];
  raw = rpbh_load_row(X, base + rs, M, K, cidx);
#pragma unroll
  for (int i = 0; i < PV; ++i) {
    const int c = min(t + 64 * RPBH_WAVES * i, (K >> 2) - 1);
    reinterpret_cast<uint2*>(tab)[c] = make_uint2((pv[i].x & 0xFFFFu) | (pv[i].y << 16),
                                                    (pv[i].z & 0xFFFFu) | (pv[i].w << 16));
  }
  {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) m |= ((sv[i] >> (8 * k + 7)) & 1u) << (4 * i + k);
    smask[sb_] = m;
  }
  const MfmaXform xf = mfma_xform_hadamard(lane);
  lds_barrier();     // the table is visible; the row loads stay in flight

  for (; base < M; base += stride) {
    const int64_t row = base + rs;
    if (WPR > 1) lds_barrier();          // the previous row's gathers are done
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < RPBH_LMAX; ++j) {
      reinterpret_cast<v4u*>(slot)[cidx[j]] = raw.v[j];    // repeated chunks rewrite identical data
      if (CENTER) {
        float x[8];
        unpack8_f16(raw.v[j], x);
        float ps = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) ps += x[m];
        const bool counted = j < nl && wr * 64 + lane + 64 * WPR * j < G;   // a repeated chunk is not
        psum += counted ? ps : 0.0f;
      }
    }
    raw = rpbh_load_row(X, row + stride, M, K, cidx);   // prefetch this wave's next row
    float tot = 0.0f;
    if (CENTER) tot = wave_sum(psum);
    if (WPR > 1) {
      if (CENTER && lane == 0) red[wid] = tot;
      lds_barrier();
      if (CENTER) {
        tot = 0.0f;
#pragma unroll
        for (int w = 0; w < WPR; ++w) tot += red[rs * WPR + w];
      }
    } else {
      // the row slot is private to this wavefront: its LDS writes complete before its
      // later LDS reads, so no barrier is needed, only no reordering by the compiler
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
    float m32 = 0.0f;
    if (CENTER) {
      const __half mh = __float2half_rn(tot / (float)K);
      m32 = 32.0f * __half2float(mh);
      if (row < M && wr == 0 && lane == 0) mu[row] = mh;
    }
    uint8_t* const crow = codes + row * (int64_t)(K >> 1);
    uint8_t* const srow_sc = scales + row * (int64_t)nb;
    // chunks wr, wr + WPR, ... of the row, two at a time
    for (int ch0 = wr; ch0 < nchunk; ch0 += 2 * WPR) {
      float y[2][8];
      int blk[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        blk[u] = 16 * (ch0 + u * WPR) + bl;
        const int bb = blk[u] < nb ? blk[u] : 0;    // lanes past the row's end gather block 0, not stored
        const uint4 ix = *reinterpret_cast<const uint4*>(tab + 32 * bb + 8 * q);
        const uint32_t iw[4] = {ix.x, ix.y, ix.z, ix.w};
        v8h b;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          b[i] = __builtin_bit_cast(_Float16, slot[(iw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu]);
        mfma_block_transform<false>(xf, b, y[u]);
        const uint32_t sm = smask[bb];
        if (CENTER && q == 0) y[u][0] -= m32;     // output 0 of the block
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = (i < 4 ? 4 * q + i : 16 + 4 * q + (i - 4));
          const float c = ((sm >> j) & 1u) ? -KQ_INV_SQRT32 : KQ_INV_SQRT32;
          y[u][i] = __builtin_fmaf(y[u][i], c, 0.0f);   // +0 for an exact zero
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t w, sb;
        int off;
        mx_pack_block(y[u], q, w, off, sb);
        if (row < M && ch0 + u * WPR < nchunk && blk[u] < nb) {
          *reinterpret_cast<uint32_t*>(crow + 16 * blk[u] + off) = w;
          if (q == 0) srow_sc[blk[u]] = (uint8_t)sb;
        }
      }
    }
  }
}

hipError_t launch_kron_mx_mfma(bool kron, const __half* X, int64_t nblocks, const KronFactors& f, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
  constexpr int U = 4;
  const int64_t nchunks = (nblocks + 15) / 16;
  const int64_t waves = (nchunks + U - 1) / U;
  int64_t grid = (waves + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  if (kron)
    hipLaunchKernelGGL((kron_mx_mfma_stream_kernel<U, true>), dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(X), nblocks, f, codes, scales);
  else
    hipLaunchKernelGGL((kron_mx_mfma_stream_kernel<U, false>), dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(X), nblocks, f, codes, scales);
  return hipGetLastError();
}

template <bool CENTER, int WPR>
static hipError_t rpbh_launch(const __half* X, int64_t M, int K, const int32_t* perm, const int8_t* sign,
                              uint8_t* codes, uint8_t* scales, __half* mu, hipStream_t s) {
  const size_t lds = rpbh_lds_bytes(WPR, K);
  // one resident wave of workgroups: as many as fit on the chip at once, at most one
  // per group of NR rows
  constexpr int NR = RPBH_WAVES / WPR;
  int64_t grid = (M + NR - 1) / NR;
  const int64_t cap = (int64_t)device_cu_count() *
                      resident_blocks_per_cu(reinterpret_cast<const void*>(&rpbh_mx_mfma_rows_kernel<CENTER, WPR>),
                                             64 * RPBH_WAVES, lds);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((rpbh_mx_mfma_rows_kernel<CENTER, WPR>), dim3((unsigned)grid), dim3(64 * RPBH_WAVES), lds, s, X,
                     M, K, perm, sign, codes, scales, mu);
  return hipGetLastError();
}

template <bool CENTER>
static hipError_t rpbh_launch_wpr(const __half* X, int64_t M, int K, const int32_t* perm, const int8_t* sign,
                                  uint8_t* codes, uint8_t* scales, __half* mu, hipStream_t s) {
  // waves per row: the fewest that keep each lane at <= RPBH_LMAX 16-byte chunks of a row
  const int G = K / 8;
  if (G <= 64 * RPBH_LMAX) return rpbh_launch<CENTER, 1>(X, M, K, perm, sign, codes, scales, mu, s);
  if (G <= 128 * RPBH_LMAX) return rpbh_launch<CENTER, 2>(X, M, K, perm, sign, codes, scales, mu, s);
  if (G <= 256 * RPBH_LMAX) return rpbh_launch<CENTER, 4>(X, M, K, perm, sign, codes, scales, mu, s);
  if (G <= 512 * RPBH_LMAX) return rpbh_launch<CENTER, 8>(X, M, K, perm, sign, codes, scales, mu, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rpbh_mx_mfma(bool center, const __half* X, int64_t M, int64_t K, const int32_t* perm,
                               const int8_t* sign, uint8_t* codes, uint8_t* scales, __half* mu, hipStream_t s) {
  if (K > 65536) return hipErrorInvalidValue;    // u16 gather indices
  return center ? rpbh_launch_wpr<true>(X, M, (int)K, perm, sign, codes, scales, mu, s)
                : rpbh_launch_wpr<false>(X, M, (int)K, perm, sign, codes, scales, mu, s);
}

int resident_blocks_per_cu(const void* kernel, int threads, size_t lds) {
  static std::mutex mtx;
  static std::map<std::tuple<const void*, int, size_t>, int> cache;
  const auto key = std::make_tuple(kernel, threads, lds);
  std::lock_guard<std::mutex> lock(mtx);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1) n = 1;
  cache.emplace(key, n);
  return n;
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

template <int KIND, int FMT, bool CENTER, int NG>
static hipError_t row_launch(unsigned threads, size_t lds, const __half* X, int64_t M, int K, const KronFactors& f,
                             const int32_t* perm, const int8_t* sign, uint8_t* codes, void* scales, __half* mu,
                             hipStream_t s) {
  // persistent workgroups (one resident wave of them): the per-row gather indices are
  // set up once per workgroup
  const auto kern = row_quant_kernel<KIND, FMT, CENTER, NG>;
  int64_t grid = M;
  const int64_t cap = (int64_t)device_cu_count() *
                      resident_blocks_per_cu(reinterpret_cast<const void*>(kern), (int)threads, lds);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, s, X, M, K, f, perm, sign, lm_tables(), codes,
                     scales, mu);
  return hipGetLastError();
}

template <int KIND, int FMT, bool CENTER>
static hipError_t row_launch_ng(int ng, unsigned threads, size_t lds, const __half* X, int64_t M, int K,
                                const KronFactors& f, const int32_t* perm, const int8_t* sign, uint8_t* codes,
                                void* scales, __half* mu, hipStream_t s) {
  switch (ng) {
    case 1: return row_launch<KIND, FMT, CENTER, 1>(threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
    case 2: return row_launch<KIND, FMT, CENTER, 2>(threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
    case 3: return row_launch<KIND, FMT, CENTER, 3>(threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
    default: return row_launch<KIND, FMT, CENTER, 4>(threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
  }
}

template <int KIND>
static hipError_t row_launch_kind(int fmt, bool center, int ng, unsigned threads, size_t lds, const __half* X,
                                  int64_t M, int K, const KronFactors& f, const int32_t* perm, const int8_t* sign,
                                  uint8_t* codes, void* scales, __half* mu, hipStream_t s) {
  if (fmt == 0) {
    return center ? row_launch_ng<KIND, 0, true>(ng, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s)
                  : row_launch_ng<KIND, 0, false>(ng, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
  }
  return center ? row_launch_ng<KIND, 1, true>(ng, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s)
                : row_launch_ng<KIND, 1, false>(ng, threads, lds, X, M, K, f, perm, sign, codes, scales, mu, s);
}

hipError_t launch_row_quant(int kind, int fmt, bool center, const __half* X, int64_t M, int64_t K,
                            const KronFactors& f, const int32_t* perm, const int8_t* sign, uint8_t* codes,
                            void* scales, __half* mu, hipStream_t s) {
  // threads per row: the smallest multiple of 64 (at most 512) that leaves each thread at
  // most 4 groups of 8 elements; small workgroups keep many rows resident per CU
  const int G = (int)(K / 8);
  unsigned threads = 64;
  while (threads < 512 && (G + threads - 1) / threads > 4) threads += 64;
  const int ng = (int)((G + threads - 1) / threads);
  if (ng > 4) return hipErrorInvalidValue;          // K > 16384 on the row path is rejected by the caller
  const size_t lds = (kind == 2 ? (size_t)K * 4 : 0) + 2 * 32 * sizeof(float);
  switch (kind) {
    case 1: return row_launch_kind<1>(fmt, center, ng, threads, lds, X, M, (int)K, f, perm, sign, codes, scales, mu, s);
    case 2: return row_launch_kind<2>(fmt, center, ng, threads, lds, X, M, (int)K, f, perm, sign, codes, scales, mu, s);
    default: return row_launch_kind<0>(fmt, center, ng, threads, lds, X, M, (int)K, f, perm, sign, codes, scales, mu, s);
  }
}

}  // namespace kq
