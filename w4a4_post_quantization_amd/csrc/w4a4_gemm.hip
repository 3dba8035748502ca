// The W4A4 linear: Y = Xq Wq^T + T L2^T + mu wbar^T, fp32 accumulation, fp16 output.
//
// KroQuant §01 / OrbitQuant §03: both operands are already in the transformed basis
// ((XP) and (P^-1 W)), so the 4-bit product needs no transform of its own.  Each pair
// of 32-element blocks contributes 2^(ex + ew) sum_k e2m1(qx) e2m1(qw), which is exactly
// what gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 computes with FP4 operands and E8M0
// scale bytes: lane l holds row l%16 and the 32 codes of k-block l/16 (16 bytes,
// element 2i in the low nibble), plus that block's scale byte.
// SVDQuant explainer §3: the low-rank branch is fused into the same kernel: the
// accumulators start from T L2^T (fp16 MFMA), so no separate pass touches Y.
// CentriQ abstract: the rank-1 term mu wbar^T restores the token means before the store.
//
// The MFMA computes C^T tiles (weight rows as the A operand, activation rows as B), so a
// lane ends with four consecutive output columns of one output row: one 8-byte store.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row, so that the 16-byte
// MFMA fragment reads (16 rows x one chunk) and the staging writes hit distinct banks.
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(WN * WM * 64) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, const uint8_t* __restrict__ xcodes,
    const uint8_t* __restrict__ xscales, int M, int N, int K, const __half* __restrict__ T,
    const __half* __restrict__ L2, int r, const __half* __restrict__ mu, const __half* __restrict__ wbar,
    __half* __restrict__ Y) {
  constexpr int NT = WN * WM * 64;
  constexpr int TN = BN / WN / 16, TM = BM / WM / 16;
  constexpr int A_OFF = 0, B_OFF = BN * 64, AS_OFF = B_OFF + BM * 64, BS_OFF = AS_OFF + BN * 4;
  constexpr int BUF = BS_OFF + BM * 4;
  constexpr int ACH = BN * 4 / NT, BCH = BM * 4 / NT;
  static_assert(ACH * NT == BN * 4 && BCH * NT == BM * 4, "tile/threads mismatch");
  __shared__ __align__(16) uint8_t lds[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid % WN, wm = wid / WN;
  const int lr = lane & 15, q = lane >> 4;

  // tile order: consecutive workgroups land on different XCDs (round-robin dispatch), so
  // renumber them so each XCD walks a contiguous range of tiles, and walk tiles in
  // groups of 8 along M to share operand rows in that XCD's L2.
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const int ntiles = tiles_n * tiles_m;
  int pid = blockIdx.x;
  {
    const int per = ntiles / 8, rem = ntiles % 8, xcd = pid % 8, loc = pid / 8;
    if (pid < 8 * per) pid = xcd * per + loc;
    (void)rem;
  }
  constexpr int GM = 8;
  const int group = pid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int tile_m = first_m + (pid % (GM * tiles_n)) % gsize;
  const int tile_n = (pid % (GM * tiles_n)) / gsize;
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  const int KB = K >> 1;   // code bytes per row
  const int KS = K >> 5;   // scale bytes per row
  const int nk = K >> 7;   // 128-wide k-steps

  // staging assignment
  const uint8_t* ga[ACH];
  int la[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + NT * i, row = c >> 2, qq = c & 3;
    const int gr = min(n0 + row, N - 1);
    ga[i] = wcodes + (int64_t)gr * KB + 16 * qq;
    la[i] = A_OFF + row * 64 + 16 * (qq ^ chunk_swz(row));
  }
  const uint8_t* gb[BCH];
  int lb[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + NT * i, row = c >> 2, qq = c & 3;
    const int gr = min(m0 + row, M - 1);
    gb[i] = xcodes + (int64_t)gr * KB + 16 * qq;
    lb[i] = B_OFF + row * 64 + 16 * (qq ^ chunk_swz(row));
  }
  // scale dwords: one per row per k-step
  const uint8_t* gsc = nullptr;
  int lsc = 0;
  if (tid < BN) {
    gsc = wscales + (int64_t)min(n0 + tid, N - 1) * KS;
    lsc = AS_OFF + tid * 4;
  } else if (tid < BN + BM) {
    gsc = xscales + (int64_t)min(m0 + tid - BN, M - 1) * KS;
    lsc = BS_OFF + (tid - BN) * 4;
  }
  static_assert(BN + BM <= NT * 2, "scale staging needs more threads");
  const uint8_t* gsc2 = nullptr;
  int lsc2 = 0;
  if (BN + BM > NT && tid + NT < BN + BM) {
    const int t2 = tid + NT;
    gsc2 = xscales + (int64_t)min(m0 + t2 - BN, M - 1) * KS;
    lsc2 = BS_OFF + (t2 - BN) * 4;
  }

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int wrow_a = wn * (BN / WN), wrow_b = wm * (BM / WM);

  // low-rank branch first: acc = T L2^T (fp16 MFMA 16x16x32, r/32 steps, r = 16 padded)
  if (r > 0) {
    for (int rc = 0; rc < r; rc += 32) {
      v8h la8[TN], lb8[TM];
      const bool live = (rc + 8 * q) < r;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int n = min(n0 + wrow_a + 16 * i + lr, N - 1);
        la8[i] = live ? *reinterpret_cast<const v8h*>(L2 + (int64_t)n * r + rc + 8 * q) : v8h{};
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = min(m0 + wrow_b + 16 * j + lr, M - 1);
        lb8[j] = live ? *reinterpret_cast<const v8h*>(T + (int64_t)m * r + rc + 8 * q) : v8h{};
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(la8[i], lb8[j], acc[i][j], 0, 0, 0);
    }
  }

  uint4 ra[ACH], rb[BCH];
  uint32_t rs = 0, rs2 = 0;
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = *reinterpret_cast<const uint4*>(ga[i] + 64 * ks);
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb[i] = *reinterpret_cast<const uint4*>(gb[i] + 64 * ks);
    if (gsc) rs = *reinterpret_cast<const uint32_t*>(gsc + 4 * ks);
    if (gsc2) rs2 = *reinterpret_cast<const uint32_t*>(gsc2 + 4 * ks);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * BUF;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<uint4*>(base + la[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *reinterpret_cast<uint4*>(base + lb[i]) = rb[i];
    if (gsc) *reinterpret_cast<uint32_t*>(base + lsc) = rs;
    if (gsc2) *reinterpret_cast<uint32_t*>(base + lsc2) = rs2;
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* base = lds + cur * BUF;
    v8i fa[TN], fb[TM];
    int sa[TN], sb[TM];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int row = wrow_a + 16 * i + lr;
      const uint4 v = *reinterpret_cast<const uint4*>(base + A_OFF + row * 64 + 16 * (q ^ chunk_swz(row)));
      fa[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      sa[i] = base[AS_OFF + row * 4 + q];
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = wrow_b + 16 * j + lr;
      const uint4 v = *reinterpret_cast<const uint4*>(base + B_OFF + row * 64 + 16 * (q ^ chunk_swz(row)));
      fb[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      sb[j] = base[BS_OFF + row * 4 + q];
    }
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
    if (ks + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: acc[i][j][e] = Y[m][n + e] with n = .. + 4q, m = .. + lr
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int n = n0 + wrow_a + 16 * i + 4 * q;
    float wb[4] = {0.f, 0.f, 0.f, 0.f};
    if (mu && n < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) wb[e] = __half2float(wbar[n + e]);
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wrow_b + 16 * j + lr;
      if (m >= M || n >= N) continue;
      v4f v = acc[i][j];
      if (mu) {
        const float mm = __half2float(mu[m]);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(mm, wb[e], v[e]);
      }
      const __half2 h0 = __floats2half2_rn(v[0], v[1]);
      const __half2 h1 = __floats2half2_rn(v[2], v[3]);
      uint2 out;
      out.x = __builtin_bit_cast(uint32_t, h0);
      out.y = __builtin_bit_cast(uint32_t, h1);
      *reinterpret_cast<uint2*>(Y + (int64_t)m * N + n) = out;
    }
  }
}

hipError_t launch_w4a4_gemm(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                            const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                            hipStream_t s) {
  constexpr int BN = 128, BM = 128, WN = 2, WM = 2;
  const int64_t tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  hipLaunchKernelGGL((w4a4_gemm_kernel<BN, BM, WN, WM>), dim3((unsigned)tiles), dim3(WN * WM * 64), 0, s, wcodes,
                     wscales, xcodes, xscales, (int)M, (int)N, (int)K, T, L2, r, mu, wbar, Y);
  return hipGetLastError();
}

}  // namespace kq
