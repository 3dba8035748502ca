// W2A4 linear for the rotated, calibration-free path (OrbitQuant §03: one Lloyd-Max
// codebook for all rotated coordinates; §04: 2-bit weights, 4-bit activations; CentriQ
// abstract: closed-form per-token scale):
//   Y[m][n] = s_t[m] * sum_g s_g[n][g] * sum_{k in g} l16[qx[m][k]] * l4[qw[n][k]].
// The codes are table-dequantized to fp16 in LDS once per workgroup tile (activation
// levels without their per-token scale, weight levels times their fp16 group scale) and
// multiplied on the fp16 matrix cores (fp32 accumulation); the per-token scale multiplies
// the accumulator before the fp16 store.  Two forms: 128 x 128 tiles of 16 x 16 x 32
// products, and 256 x 256 tiles of 32 x 32 x 16 products for grids of at least 1.5 rounds.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

__device__ __forceinline__ int chunk_swz2(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Dequantization tables in LDS, entry b for a byte of codes: lut16[b] = the fp16 levels of
// its two 4-bit codes (low nibble first; bit 3 the sign), lut4[b] = those of its four 2-bit
// codes (low pair first; bit 1 the sign).  Threads tid, tid + nt, ... fill the entries.
__device__ __forceinline__ void build_lm_luts(const LmTables& lm, uint32_t* lut16, uint2* lut4, int tid, int nt) {
  for (int b = tid; b < 256; b += nt) {
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
}

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

  build_lm_luts(lm, lut16, lut4, tid, NT);

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

// Large-tile form: BN = 256 weight rows x BM = 256 tokens per workgroup on 4 wavefronts
// (2 x 2), each owning a 128 x 128 block of 32 x 32 output tiles
// (v_mfma_f32_32x32x16_f16: lane l holds row l % 32 and k = 8 (l / 32) .. + 7 of each
// 16-wide step; result register 4 g + e of lane l is C[8 g + 4 (l / 32) + e][l % 32]).
// Against 64 x 64 wave tiles of 16 x 16 products this reads half the LDS bytes per
// product.  A k-step is two groups (64 k): a barrier then separates 64 products per
// wavefront, and the global loads of the next step, issued before them, have that long
// to land.  Thread t stages weight row t and token row t; LDS rows are 128 bytes, their
// 16-byte chunks XOR-swizzled by the row's low bits.
// What bounds it is LDS: per step the compute unit reads 128 KiB of fragments, makes
// 12 K table lookups at random addresses and stores 64 KiB, about as long as the step's
// matrix-core work.
// A last step with one group left (K % 64 = 32) leaves the other group's values zero.
__global__ __launch_bounds__(256, 1) void w2a4_gemm_big_kernel(
    const uint8_t* __restrict__ xcodes, const float* __restrict__ xscales, int M, int K,
    const uint8_t* __restrict__ wcodes, const __half* __restrict__ wscales, int N, LmTables lm,
    __half* __restrict__ Y) {
  constexpr int BN = 256, BM = 256, TN = 4, TM = 4, RB = 128;   // RB: LDS bytes per row and step
  constexpr int A_OFF = 0, B_OFF = BN * RB, BUF = (BN + BM) * RB;
  __shared__ __align__(16) uint8_t lds[2 * BUF];
  __shared__ uint32_t lut16[256];   // byte of two 4-bit codes -> two fp16 levels
  __shared__ uint2 lut4[256];       // byte of four 2-bit codes -> four fp16 levels

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int l32 = lane & 31, h = lane >> 5;

  build_lm_luts(lm, lut16, lut4, tid, 256);

  // tiles walked column by column in groups of 8 along M, die-contiguous (as the W4A4 form)
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const int ntiles = tiles_n * tiles_m;
  int pid = blockIdx.x;
  {
    const int per = ntiles / 8;
    if (pid < 8 * per) pid = (pid % 8) * per + pid / 8;
  }
  constexpr int GM = 8;
  const int group = pid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int tile_m = first_m + (pid % (GM * tiles_n)) % gsize;
  const int tile_n = (pid % (GM * tiles_n)) / gsize;
  const int n0 = tile_n * BN, m0 = tile_m * BM;
  const int ng = K >> 5, nks = (ng + 1) >> 1;             // groups, 64-wide steps

  // staging rows of this thread: weight row tid, token row tid; rows past the matrix repeat
  // its last row (their results are never stored)
  const int64_t wrow = min(n0 + tid, N - 1), xrow = min(m0 + tid, M - 1);
  const uint8_t* const gw = wcodes + wrow * (K >> 2);
  const __half* const gs = wscales + wrow * (K >> 5);
  const uint8_t* const gx = xcodes + xrow * (K >> 1);
  const int sw = tid & 7;

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  uint2 rw[2];      // codes of the step's two groups (8 bytes each)
  __half sg[2];
  uint4 rx[2];      // ... 16 bytes each
  auto gload = [&](int ks) {
    const bool two = 2 * ks + 1 < ng;                      // the step's second group exists
    rw[0] = *reinterpret_cast<const uint2*>(gw + 16 * ks);
    sg[0] = gs[2 * ks];
    rw[1] = two ? *reinterpret_cast<const uint2*>(gw + 16 * ks + 8) : make_uint2(0u, 0u);
    sg[1] = two ? gs[2 * ks + 1] : __float2half(0.0f);     // a zero scale zeroes the group
    rx[0] = *reinterpret_cast<const uint4*>(gx + 32 * ks);
    rx[1] = two ? *reinterpret_cast<const uint4*>(gx + 32 * ks + 16) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto lstore = [&](int buf, bool two) {
    uint8_t* const base = lds + buf * BUF;
#pragma unroll
    for (int q = 0; q < 2; ++q) {                          // group q: chunks 4 q .. 4 q + 3
      const __half2 s2 = __half2half2(sg[q]);
      const uint32_t wv[2] = {rw[q].x, rw[q].y};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t hw[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int bI = 2 * c + u;
          const uint2 pr = lut4[(wv[bI >> 2] >> (8 * (bI & 3))) & 0xFF];
          hw[2 * u] = __builtin_bit_cast(uint32_t, __hmul2(__builtin_bit_cast(__half2, pr.x), s2));
          hw[2 * u + 1] = __builtin_bit_cast(uint32_t, __hmul2(__builtin_bit_cast(__half2, pr.y), s2));
        }
        *reinterpret_cast<uint4*>(base + A_OFF + tid * RB + 16 * ((4 * q + c) ^ sw)) =
            make_uint4(hw[0], hw[1], hw[2], hw[3]);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t xv[4] = {rx[q].x, rx[q].y, rx[q].z, rx[q].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t hx[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int bI = 4 * c + u;
          hx[u] = (q == 0 || two) ? lut16[(xv[bI >> 2] >> (8 * (bI & 3))) & 0xFF] : 0u;
        }
        *reinterpret_cast<uint4*>(base + B_OFF + tid * RB + 16 * ((4 * q + c) ^ sw)) =
            make_uint4(hx[0], hx[1], hx[2], hx[3]);
      }
    }
  };

  const int wrow_a = wn * 128, wrow_b = wm * 128;
  gload(0);
  __syncthreads();  // tables ready
  lstore(0, 1 < ng);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    if (ks + 1 < nks) gload(ks + 1);
    const uint8_t* const base = lds + (ks & 1) * BUF;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {       // four 16-wide steps: chunks 2 sub + (l / 32)
      const int ch = 2 * sub + h;
      v8h fa[TN], fb[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int row = wrow_a + 32 * i + l32;
        fa[i] = *reinterpret_cast<const v8h*>(base + A_OFF + row * RB + 16 * (ch ^ (row & 7)));
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int row = wrow_b + 32 * j + l32;
        fb[j] = *reinterpret_cast<const v8h*>(base + B_OFF + row * RB + 16 * (ch ^ (row & 7)));
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nks) lstore((ks + 1) & 1, 2 * (ks + 1) + 1 < ng);
    __syncthreads();
  }

  // acc[i][j][4 g + e] = (unscaled) Y[m][n] for m = m0 + wrow_b + 32 j + l % 32,
  // n = n0 + wrow_a + 32 i + 8 g + 4 (l / 32) + e: one 8-byte store per (i, j, g)
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + wrow_b + 32 * j + l32;
    if (m >= M) continue;
    const float st = xscales[m];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wrow_a + 32 * i + 8 * g + 4 * h;
        if (n >= N) continue;
        const v16f& v = acc[i][j];
        const __half2 h0 = __floats2half2_rn(v[4 * g] * st, v[4 * g + 1] * st);
        const __half2 h1 = __floats2half2_rn(v[4 * g + 2] * st, v[4 * g + 3] * st);
        *reinterpret_cast<uint2*>(Y + (int64_t)m * N + n) =
            make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
      }
  }
}

hipError_t launch_w2a4_gemm(const uint8_t* xcodes, const float* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const __half* wscales, int64_t N, __half* Y, hipStream_t s) {
  // The large-tile form does a 256 x 256 tile in about 0.7 of the time of four 128 x 128
  // ones, but its rounds of tiles are four times coarser: it measured faster at 1.7 rounds
  // (SANA-like qkv: 232 vs 289 us) and slower at 1.4 and 0.6 (fc1: 220 vs 211, fc2: 256 vs
  // 223), so it runs from 1.5 rounds up.
  const int64_t cus = device_cu_count();
  const int64_t t256 = ((N + 255) / 256) * ((M + 255) / 256);
  if (2 * t256 >= 3 * cus) {
    hipLaunchKernelGGL(w2a4_gemm_big_kernel, dim3((unsigned)t256), dim3(256), 0, s, xcodes, xscales, (int)M,
                       (int)K, wcodes, wscales, (int)N, lm_tables(), Y);
    return hipGetLastError();
  }
  constexpr int BN = 128, BM = 128, WN = 2, WM = 2;
  const int64_t tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  hipLaunchKernelGGL((w2a4_gemm_kernel<BN, BM, WN, WM>), dim3((unsigned)tiles), dim3(WN * WM * 64), 0, s, xcodes,
                     xscales, (int)M, (int)K, wcodes, wscales, (int)N, lm_tables(), Y);
  return hipGetLastError();
}

}  // namespace kq
