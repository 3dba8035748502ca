// Matrix-core building blocks shared by the transform kernels and the fused low-rank
// kernel: the 32-element block transform as fp16 MFMAs, MXFP4 packing of its outputs, and
// the power-of-two channel shift.
#pragma once
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

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
// p is made opaque before it is split: otherwise the compiler rounds the lo part's hi
// straight from the exact product (v_fma_mix, one rounding) but the hi fragment from the
// float32 product (two roundings), and where the float32 product sits exactly between two
// fp16 values the two differ by one fp16 step, so hi + lo misses p by that step.
__device__ __forceinline__ MfmaXform mfma_xform_kron(const KronFactors& f, int lane) {
  MfmaXform x;
  const int q = lane >> 4, jl = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * t + jl;                 // output index (column of P)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * q + i;                 // input index (row of P)
      float p = f.A[4 * (k >> 3) + (j >> 3)] * f.B[8 * (k & 7) + (j & 7)];
      asm volatile("" : "+v"(p));
      const _Float16 hi = (_Float16)p;
      x.a[t][0][i] = hi;
      x.a[t][1][i] = (_Float16)(p - (float)hi);
    }
  }
  return x;
}

// The same fragments from one block's factors in device memory (ab = {A 4x4, B 8x8},
// row-major): each lane reads only the two A and eight B entries its fragments use.
__device__ __forceinline__ MfmaXform mfma_xform_kron_g(const float* __restrict__ ab, int lane) {
  MfmaXform x;
  const int q = lane >> 4, jl = lane & 15;
  float a[2], b[8];
#pragma unroll
  for (int t = 0; t < 2; ++t) a[t] = ab[4 * q + 2 * t + (jl >> 3)];      // A[k >> 3][j >> 3], k = 8q + i
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = ab[16 + 8 * i + (jl & 7)];           // B[k & 7][j & 7]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float p = a[t] * b[i];
      asm volatile("" : "+v"(p));                // see mfma_xform_kron
      const _Float16 hi = (_Float16)p;
      x.a[t][0][i] = hi;
      x.a[t][1][i] = (_Float16)(p - (float)hi);
    }
  return x;
}

// The same fragments for a dense 32x32 P (row-major in device memory): P^T rows j, columns k.
__device__ __forceinline__ MfmaXform mfma_xform_dense(const float* __restrict__ P, int lane) {
  MfmaXform x;
  const int q = lane >> 4, jl = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = 16 * t + jl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = P[32 * (8 * q + i) + j];   // P[k][j], k = 8q + i
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

// Per-token Lloyd-Max codes of the lane's eight outputs (same lanes and byte layout as
// mx_pack_block): 4-bit sign-magnitude, magnitude = number of the scaled thresholds ts[]
// (ascending) strictly below |y| (a value on a threshold takes the smaller magnitude),
// found by a three-step binary search; sign bit for y < 0.  Inputs must not be -0.0.
__device__ __forceinline__ void lm_pack_block(const float* y, int q, const float* ts, uint32_t& dword, int& byte_off) {
  uint32_t h[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // three-level search over the seven sorted thresholds; each level's threshold is
    // selected by the earlier levels' outcomes
    const float a = fabsf(y[i]);
    const bool c2 = a > ts[3];
    const float tm = c2 ? ts[5] : ts[1];
    const bool c1 = a > tm;
    const float tl0 = c1 ? ts[2] : ts[0], tl1 = c1 ? ts[6] : ts[4];
    const float tl = c2 ? tl1 : tl0;
    const bool c0 = a > tl;
    const uint32_t idx = (c2 ? 4u : 0u) | (c1 ? 2u : 0u) | (c0 ? 1u : 0u);
    h[i >> 2] |= (idx | (y[i] < 0.0f ? 8u : 0u)) << (4 * (i & 3));
  }
  // outputs 4q..4q+3 are bytes 2q, 2q+1 of the block; 16+4q..16+4q+3 bytes 8+2q, 8+2q+1
  const auto sw = __builtin_amdgcn_permlane16_swap(h[0], h[1], false, false);
  dword = sw[0] | (sw[1] << 16);
  byte_off = (q & 1) ? 8 + 2 * (q - 1) : 2 * q;
}

// Eight fp16 values divided by 2^e (one exponent byte each, in order): v_ldexp_f16 rounds a
// result below the normal range to nearest even, like a conversion would.
__device__ __forceinline__ uint32_t pts_scale2(uint32_t x2, uint32_t e2) {
  const _Float16 lo = __builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)(x2 & 0xFFFFu)),
                                              -(int)(e2 & 0xFFu));
  const _Float16 hi = __builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)(x2 >> 16)),
                                              -(int)((e2 >> 8) & 0xFFu));
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
__device__ __forceinline__ uint4 pts_scale8(uint4 x, uint2 e) {
  return make_uint4(pts_scale2(x.x, e.x), pts_scale2(x.y, e.x >> 16), pts_scale2(x.z, e.y), pts_scale2(x.w, e.y >> 16));
}

}  // namespace kq
