// W2A4 linear for the rotated, calibration-free path (OrbitQuant §03: one Lloyd-Max
// codebook for all rotated coordinates; §04: 2-bit weights, 4-bit activations; CentriQ
// abstract: closed-form per-token scale):
//   Y[m][n] = s_t[m] * sum_g s_g[n][g] * sum_{k in g} l16[qx[m][k]] * l4[qw[n][k]].
// The codes are table-dequantized to fp16 in LDS once per workgroup tile (activation
// levels without their per-token scale, weight levels times their fp16 group scale) and
// multiplied on the fp16 matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation);
// the per-token scale multiplies the accumulator before the fp16 store.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

__device__ __forceinline__ int chunk_swz2(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(WN * WM * 64) void w2a4_gemm_kernel(
    const uint8_t* __restrict__ xcodes, const float* __restrict__ xscales, int M, int K,
    const uint8_t* __restrict__ wcodes, const __half* __restrict__ wscales, int N, LmTables lm,
    __half* __restrict__ Y) {
  constexpr int NT = WN * WM * 64;
  constexpr int TN = BN / WN / 16, TM = BM / WM / 16;
  static_assert(BN + BM == NT, "one staging row per thread");
  constexpr int A_OFF = 0, B_OFF = BN * 64, BUF = (BN + BM) * 64;
  __shared__ __align__(16) uint8_t lds[2 * BUF];
  __shared__ uint32_t lut16[256];   // byte of two 4-bit codes -> two fp16 levels
  __shared__ uint2 lut4[256];       // byte of four 2-bit codes -> four fp16 levels

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid % WN, wm = wid / WN;
  const int lr = lane & 15, q = lane >> 4;

  // build the tables: 4-bit sign-magnitude (bit 3 sign), 2-bit sign-magnitude (bit 1 sign)
  for (int b = tid; b < 256; b += NT) {
    const int c0 = b & 15, c1 = b >> 4;
    const float v0 = (c0 & 8) ? -lm.l16[c0 & 7] : lm.l16[c0 & 7];
    const float v1 = (c1 & 8) ? -lm.l16[c1 & 7] : lm.l16[c1 & 7];
    lut16[b] = __builtin_bit_cast(uint32_t, __floats2half2_rn(v0, v1));
    float w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = (b >> (2 * e)) & 3;
      w[e] = (c & 2) ? -lm.l4[c & 1] : lm.l4[c & 1];
    }
    lut4[b] = make_uint2(__builtin_bit_cast(uint32_t, __floats2half2_rn(w[0], w[1])),
                         __builtin_bit_cast(uint32_t, __floats2half2_rn(w[2], w[3])));
  }

  const int tiles_n = (N + BN - 1) / BN;
  const int tile_n = blockIdx.x % tiles_n, tile_m = blockIdx.x / tiles_n;
  const int n0 = tile_n * BN, m0 = tile_m * BM;
  const int nk = K >> 5;

  // staging row of this thread
  const bool is_w = tid < BN;
  const int srow = is_w ? tid : tid - BN;
  const int64_t grow = is_w ? min(n0 + srow, N - 1) : min(m0 + srow, M - 1);
  const uint8_t* gcode = is_w ? wcodes + grow * (K >> 2) : xcodes + grow * (K >> 1);
  const __half* gscale = wscales + grow * (K >> 5);
  const int lrow = (is_w ? A_OFF : B_OFF) + srow * 64;
  const int sw = chunk_swz2(srow);

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 raw;
  __half sg;
  auto gload = [&](int ks) {
    if (is_w) {
      const uint2 v = *reinterpret_cast<const uint2*>(gcode + 8 * ks);
      raw = make_uint4(v.x, v.y, 0u, 0u);
      sg = gscale[ks];
    } else {
      raw = *reinterpret_cast<const uint4*>(gcode + 16 * ks);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * BUF + lrow;
    uint32_t h[16];
    if (is_w) {
      const __half2 s2 = __half2half2(sg);
      const uint32_t wv[2] = {raw.x, raw.y};
#pragma unroll
      for (int bI = 0; bI < 8; ++bI) {
        const uint2 p = lut4[(wv[bI >> 2] >> (8 * (bI & 3))) & 0xFF];
        h[2 * bI] = __builtin_bit_cast(uint32_t, __hmul2(__builtin_bit_cast(__half2, p.x), s2));
        h[2 * bI + 1] = __builtin_bit_cast(uint32_t, __hmul2(__builtin_bit_cast(__half2, p.y), s2));
      }
    } else {
      const uint32_t xv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int bI = 0; bI < 16; ++bI) h[bI] = lut16[(xv[bI >> 2] >> (8 * (bI & 3))) & 0xFF];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint4*>(base + 16 * (c ^ sw)) = make_uint4(h[4 * c], h[4 * c + 1], h[4 * c + 2], h[4 * c + 3]);
  };

  const int wrow_a = wn * (BN / WN), wrow_b = wm * (BM / WM);
  __syncthreads();  // tables ready
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* base = lds + cur * BUF;
    v8h fa[TN], fb[TM];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int row = wrow_a + 16 * i + lr;
      fa[i] = *reinterpret_cast<const v8h*>(base + A_OFF + row * 64 + 16 * (q ^ chunk_swz2(row)));
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = wrow_b + 16 * j + lr;
      fb[j] = *reinterpret_cast<const v8h*>(base + B_OFF + row * 64 + 16 * (q ^ chunk_swz2(row)));
    }
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    if (ks + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int n = n0 + wrow_a + 16 * i + 4 * q;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wrow_b + 16 * j + lr;
      if (m >= M || n >= N) continue;
      const float st = xscales[m];
      const v4f v = acc[i][j];
      const __half2 h0 = __floats2half2_rn(v[0] * st, v[1] * st);
      const __half2 h1 = __floats2half2_rn(v[2] * st, v[3] * st);
      *reinterpret_cast<uint2*>(Y + (int64_t)m * N + n) =
          make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
    }
  }
}

hipError_t launch_w2a4_gemm(const uint8_t* xcodes, const float* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const __half* wscales, int64_t N, __half* Y, hipStream_t s) {
  constexpr int BN = 128, BM = 128, WN = 2, WM = 2;
  const int64_t tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  hipLaunchKernelGGL((w2a4_gemm_kernel<BN, BM, WN, WM>), dim3((unsigned)tiles), dim3(WN * WM * 64), 0, s, xcodes,
                     xscales, (int)M, (int)K, wcodes, wscales, (int)N, lm_tables(), Y);
  return hipGetLastError();
}

}  // namespace kq
