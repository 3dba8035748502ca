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
//
// Pipeline per 128-wide k-step (64 code bytes + 4 scale bytes per row):
//   global -> registers two k-steps ahead (two staging sets, ping-pong),
//   registers -> LDS one k-step ahead (two LDS buffers),
//   LDS -> MFMA fragments for the current k-step.
// Barriers fence only LDS, so the global prefetch stays in flight across them.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row, so that the 16-byte
// MFMA fragment reads (16 rows x one chunk) and the staging writes hit distinct banks.
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

typedef int v4i __attribute__((ext_vector_type(4)));


// Tile configuration: BN weight rows x BM activation rows per workgroup, WN x WM
// wavefronts, each owning a (BN/WN) x (BM/WM) block of 32x32 MFMA tiles.  PF = how many
// k-steps ahead the global loads run (1 or 2 register staging sets).
//
// The 32x32x64 form of the scaled FP4 MFMA is the one that runs at the doubled FP4 rate
// on gfx950 (the 16x16x128 form issues at the FP8 rate).  Its operand layout: lane l
// holds row l%32 and k-block l/32 of the 64-wide k-slice (16 bytes = 32 codes) plus that
// block's E8M0 byte; the 32x32 result sits in 16 registers, register 4g+i of lane l being
// C[8g + 4(l/32) + i][l%32].
template <int BN_, int BM_, int WN_, int WM_, int PF_>
struct GemmCfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_, PF = PF_;
  static constexpr int NT = 64 * WN * WM;
  static constexpr int TN = BN / WN / 32, TM = BM / WM / 32;
  static constexpr int ACH = BN * 4 / NT, BCH = BM * 4 / NT;   // 16-byte code chunks per thread
  static constexpr int A_OFF = 0, B_OFF = BN * 64, AS_OFF = B_OFF + BM * 64, BS_OFF = AS_OFF + BN * 4;
  static constexpr int DUMMY_OFF = BS_OFF + BM * 4;             // scale slots of threads owning no row
  static constexpr int BUF = DUMMY_OFF + NT * 4;
  static_assert(ACH * NT == BN * 4 && BCH * NT == BM * 4, "tile rows x 4 chunks must spread over the threads");
  static_assert(BN <= NT && BM <= NT, "one scale dword per thread per operand");
  static_assert(TN >= 1 && TM >= 1, "wave tile too small");
};

template <class C>
struct GemmStage {
  v4i a[C::ACH], b[C::BCH];
  int sa, sb;
};

template <class C, bool LR, bool MU>
__global__ __launch_bounds__(C::NT) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, const uint8_t* __restrict__ xcodes,
    const uint8_t* __restrict__ xscales, int M, int N, int K, const __half* __restrict__ T,
    const __half* __restrict__ L2, int r, const __half* __restrict__ mu, const __half* __restrict__ wbar,
    __half* __restrict__ Y) {
  using S = GemmStage<C>;
  constexpr int NT = C::NT, ACH = C::ACH, BCH = C::BCH, TN = C::TN, TM = C::TM, BN = C::BN, BM = C::BM;
  __shared__ __align__(16) uint8_t lds[2 * C::BUF];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid % C::WN, wm = wid / C::WN;
  const int l32 = lane & 31, h = lane >> 5;

  // tile order: workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // each XCD walks a contiguous range of tiles, grouped 8 deep along M so neighbouring
  // tiles share operand rows in that XCD's L2.
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

  const int KB = K >> 1;   // code bytes per row
  const int KS = K >> 5;   // scale bytes per row
  const int nk = K >> 7;   // 128-wide k-steps

  // operand windows of this tile (rows past N or M read as zeros)
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(wcodes + (int64_t)n0 * KB, (int64_t)(N - n0) * KB);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(xcodes + (int64_t)m0 * KB, (int64_t)(M - m0) * KB);
  const __amdgpu_buffer_rsrc_t rAS = make_rsrc(wscales + (int64_t)n0 * KS, (int64_t)(N - n0) * KS);
  const __amdgpu_buffer_rsrc_t rBS = make_rsrc(xscales + (int64_t)m0 * KS, (int64_t)(M - m0) * KS);

  // staging assignment: 16-byte chunk c = tid + NT*i is row c/4, chunk c%4
  int oa[ACH], la[ACH], ob[BCH], lb[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + NT * i, row = c >> 2, qq = c & 3;
    oa[i] = row * KB + 16 * qq;
    la[i] = C::A_OFF + row * 64 + 16 * (qq ^ chunk_swz(row));
  }
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + NT * i, row = c >> 2, qq = c & 3;
    ob[i] = row * KB + 16 * qq;
    lb[i] = C::B_OFF + row * 64 + 16 * (qq ^ chunk_swz(row));
  }
  // scale dwords: thread t < BN (< BM) stages row t's; the others read past the window
  // (zeros) and store into a dummy slot, so the loop body has no branches
  const int osa = tid * KS, osb = tid * KS;
  const int lsa = tid < BN ? C::AS_OFF + 4 * tid : C::DUMMY_OFF + 4 * tid;
  const int lsb = tid < BM ? C::BS_OFF + 4 * tid : C::DUMMY_OFF + 4 * tid;
  const int sa_ok = tid < BN, sb_ok = tid < BM;

  auto gload = [&](S& st, int ks) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, oa[i], 64 * ks, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i) st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, ob[i], 64 * ks, 0);
    st.sa = __builtin_amdgcn_raw_buffer_load_b32(rAS, sa_ok ? osa : 0x7FFFFFF0, 4 * ks, 0);
    st.sb = __builtin_amdgcn_raw_buffer_load_b32(rBS, sb_ok ? osb : 0x7FFFFFF0, 4 * ks, 0);
  };
  auto lstore = [&](const S& st, int buf) {
    uint8_t* base = lds + buf * C::BUF;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<v4i*>(base + la[i]) = st.a[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *reinterpret_cast<v4i*>(base + lb[i]) = st.b[i];
    *reinterpret_cast<int*>(base + lsa) = st.sa;
    *reinterpret_cast<int*>(base + lsb) = st.sb;
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wrow_a = wn * (BN / C::WN), wrow_b = wm * (BM / C::WM);

  S st0, st1;
  gload(st0, 0);
  if (C::PF == 2) gload(st1, 1);

  // low-rank branch while the first k-steps are in flight: acc = T L2^T, fp16 MFMA
  // 32x32x16 (lane l: row l%32, k = 8(l/32)..+7), r/16 steps
  if (LR) {
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(T + (int64_t)m0 * r, (int64_t)(M - m0) * r * 2);
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(L2 + (int64_t)n0 * r, (int64_t)(N - n0) * r * 2);
    for (int rc = 0; rc < r; rc += 16) {
      v8h lb8[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j)
        lb8[j] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rT, ((wrow_b + 32 * j + l32) * r + rc + 8 * h) * 2, 0, 0));
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const v8h la8 = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rL, ((wrow_a + 32 * i + l32) * r + rc + 8 * h) * 2, 0, 0));
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(la8, lb8[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  lstore(st0, 0);
  lds_barrier();

  // one 128-wide k-step = two 64-wide MFMA slices; slice s uses chunk 2s + (l/32)
  auto compute = [&](int buf) {
    const uint8_t* base = lds + buf * C::BUF;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ch = 2 * sl + h;
      v8i fb[TM];
      int sb[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int row = wrow_b + 32 * j + l32;
        const v4i v = *reinterpret_cast<const v4i*>(base + C::B_OFF + row * 64 + 16 * (ch ^ chunk_swz(row)));
        fb[j] = v8i{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        sb[j] = base[C::BS_OFF + row * 4 + ch];
      }
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int row = wrow_a + 32 * i + l32;
        const v4i v = *reinterpret_cast<const v4i*>(base + C::A_OFF + row * 64 + 16 * (ch ^ chunk_swz(row)));
        const v8i fa = v8i{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        const int sa = base[C::AS_OFF + row * 4 + ch];
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[j], acc[i][j], 4, 4, 0, sa, 0, sb[j]);
      }
    }
  };

  // The scheduling fences keep the order load-issue / MFMAs / LDS stores: the stores wait
  // for their global loads, and hoisting them above the MFMAs would expose the whole
  // load latency on every k-step.  Loads past the last k-step read past the operand window
  // or into the next row and are never consumed.
  if (C::PF == 2) {
    // two k-steps per trip so the staging sets alternate without register copies:
    // entering a trip, LDS buffer 0 holds k-step ks and st1 holds ks+1 (possibly in flight)
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
      gload(st0, ks + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
      __builtin_amdgcn_sched_barrier(0);
      lstore(st1, 1);
      lds_barrier();
      gload(st1, ks + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
      __builtin_amdgcn_sched_barrier(0);
      lstore(st0, 0);
      lds_barrier();
    }
    if (ks < nk) compute(0);   // odd number of k-steps: the last one sits in buffer 0
  } else {
    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      gload(st0, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(cur);
      __builtin_amdgcn_sched_barrier(0);
      lstore(st0, cur ^ 1);
      lds_barrier();
    }
  }

  // ---- epilogue: acc[i][j][4g+e] = Y[m][n + e] with n = .. + 8g + 4(l/32), m = .. + l%32
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(Y + (int64_t)m0 * N, (int64_t)(M - m0) * N * 2);
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int ml = wrow_b + 32 * j + l32;            // row within the tile
    const float mm = MU ? __half2float(mu[min(m0 + ml, M - 1)]) : 0.0f;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wrow_a + 32 * i + 8 * g + 4 * h;   // column within the tile
        const bool ncol = n0 + nl < N;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
        if (MU) {
          const int nn = ncol ? n0 + nl : 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(mm, __half2float(wbar[nn + e]), v[e]);
        }
        const __half2 h0 = __floats2half2_rn(v[0], v[1]);
        const __half2 h1 = __floats2half2_rn(v[2], v[3]);
        const int off = ncol ? (ml * N + n0 + nl) * 2 : 0x7FFFFFF0;   // rows past M fall off the buffer
        const v2u outv = {__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
        __builtin_amdgcn_raw_buffer_store_b64(outv, rY, off, 0, 0);
      }
    }
  }
}

template <class C>
static hipError_t gemm_launch(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                              const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                              const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                              hipStream_t s) {
  const int64_t tiles = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
  const dim3 g((unsigned)tiles), b(C::NT);
  if (r > 0 && mu)
    hipLaunchKernelGGL((w4a4_gemm_kernel<C, true, true>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  else if (r > 0)
    hipLaunchKernelGGL((w4a4_gemm_kernel<C, true, false>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  else if (mu)
    hipLaunchKernelGGL((w4a4_gemm_kernel<C, false, true>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  else
    hipLaunchKernelGGL((w4a4_gemm_kernel<C, false, false>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  return hipGetLastError();
}

#ifndef KQ_GEMM_TUNING
hipError_t launch_w4a4_gemm(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                            const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                            hipStream_t s) {
  using Big = GemmCfg<256, 256, 2, 4, 1>;
  using Small = GemmCfg<128, 128, 2, 2, 1>;
  const int64_t big_tiles = ((N + 255) / 256) * ((M + 255) / 256);
  if (big_tiles >= device_cu_count() / 2)
    return gemm_launch<Big>(xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, s);
  return gemm_launch<Small>(xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, s);
}
#endif

}  // namespace kq
