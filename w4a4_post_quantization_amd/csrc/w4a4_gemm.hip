// The W4A4 linear: Y = Xq Wq^T + T L2^T + mu wbar^T, fp32 accumulation, fp16 output.
//
// KroQuant §01 / OrbitQuant §03: both operands are already in the transformed basis
// ((XP) and (P^-1 W)), so the 4-bit product needs no transform of its own.  Each pair
// of 32-element blocks contributes 2^(ex + ew) sum_k e2m1(qx) e2m1(qw), which is exactly
// what gfx950's scaled FP4 MFMA computes from E2M1 codes (element 2i in the low nibble of
// byte i) and E8M0 scale bytes.
// SVDQuant explainer §3: the low-rank branch is fused into the same kernel: the
// accumulators start from T L2^T (fp16 MFMA), so no separate pass touches Y.
// CentriQ abstract: the rank-1 term mu wbar^T restores the token means before the store.
//
// The MFMA computes C^T tiles (weight rows as the A operand, activation rows as B), so a
// lane ends with four consecutive output columns of one output row: one 8-byte store.
//
// Two kernel forms share that arithmetic:
//   - a configurable-tile form that stages the operands global -> registers -> LDS, for
//     small grids;
//   - a 256x256-tile form whose operands go from global memory straight into LDS (buffer
//     loads with the LDS destination), four stages deep, for the large shapes.
// Per 128-wide k-step a row contributes 64 code bytes and 4 scale bytes.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row, so that the 16-byte
// MFMA fragment reads (16 rows x one chunk) and the staging writes hit distinct banks.
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }



// Configurable-tile form.  BN weight rows x BM activation rows per workgroup, WN x WM
// wavefronts, each owning a (BN/WN) x (BM/WM) block of 32x32 MFMA tiles.  PF = how many
// k-steps ahead the global loads run (1 or 2 register staging sets); registers go to LDS
// one k-step ahead (two LDS buffers), and barriers fence only LDS, so the global
// prefetch stays in flight across them.
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

  // every offset goes through the range-checked vector offset; k-steps past the last one
  // (prefetched by the pipeline, never consumed) read as zeros
  auto gload = [&](S& st, int ks) {
    const bool kv = ks < nk;
#pragma unroll
    for (int i = 0; i < ACH; ++i) st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, kv ? oa[i] + 64 * ks : KQ_OOB, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i) st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, kv ? ob[i] + 64 * ks : KQ_OOB, 0, 0);
    st.sa = __builtin_amdgcn_raw_buffer_load_b32(rAS, (sa_ok && kv) ? osa + 4 * ks : KQ_OOB, 0, 0);
    st.sb = __builtin_amdgcn_raw_buffer_load_b32(rBS, (sb_ok && kv) ? osb + 4 * ks : KQ_OOB, 0, 0);
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
  // load latency on every k-step.  Loads past the last k-step take the out-of-range offset
  // (they return zeros) and are never consumed.
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

// ---------------------------------------------------------------------------------
// Large-tile form: 256x256 tiles on 4 wavefronts (2 x 2), each owning a 128 x 128 block of
// 4 x 4 MFMA tiles (256 fp32 accumulators per lane, held in the accumulation registers),
// which halves the LDS bytes read per MFMA against 128 x 64 wave tiles.  Per 128-wide
// k-step the workgroup stages 32 KiB of codes; the fragments of the next 64-wide slice
// are read while the current slice's MFMAs run, so a single barrier per k-step suffices.
// Scale bytes are read as one dword per row and k-step: lane l shifts it by 8 (l / 32)
// and the MFMA's byte select picks block 2 s + l / 32.
struct Tile256 {
  static constexpr int BN = 256, BM = 256, NT = 256, TN = 4, TM = 4;
};

// FP4 MFMA operand from 16 code bytes: the FP4 form reads only the first four registers.
__device__ __forceinline__ v8i fp4_operand(const v4i& v) { return v8i{v.x, v.y, v.z, v.w, 0, 0, 0, 0}; }

// ---------------------------------------------------------------------------------
// The operands go from HBM straight into LDS (buffer loads with the LDS
// destination), so staging needs no registers and no LDS store instructions; four code
// stages keep three k-steps of loads in flight.  A load instruction writes 64 lanes x 16
// bytes to consecutive LDS bytes; lane L of the instruction that fills rows
// 16 q .. 16 q + 15 fetches the global chunk that the swizzled layout expects at slot L
// (row 16 q + L / 4, chunk (L % 4) ^ swizzle(row)).  Scales come in groups of four
// k-steps: one 16-byte load per row (a lane per row) into a double-buffered scale area,
// so their loads touch a fraction of the cache lines that per-k-step dword loads would.
// All offsets go in the range-checked vector offset.
// The loads are issued from inline assembly: the compiler's wait insertion would
// otherwise wait for every outstanding LDS load before each LDS read.  The kernel waits
// itself (at k-step ks, for the code loads of ks + 1; at most 16 younger loads of this
// wave are then outstanding), and one barrier per k-step makes every wave's loads visible
// and frees the stage that the next loads refill.
constexpr int DMA_STAGES = 4;
constexpr int DMA_CODE_LOADS = 8;   // code load instructions per wave per k-step
constexpr int DMA_STAGE_BYTES = Tile256::BN * 64 + Tile256::BM * 64;                  // 32 KiB of codes
constexpr int DMA_SC_OFF = DMA_STAGES * DMA_STAGE_BYTES;                       // scale groups
constexpr int DMA_SC_BYTES = (Tile256::BN + Tile256::BM) * 16;                        // one group, both operands
constexpr int DMA_MU_OFF = DMA_SC_OFF + 2 * DMA_SC_BYTES;                     // wbar of the tile
constexpr int DMA_LDS = DMA_MU_OFF + 1024;   // 148480 bytes (the wbar load writes 64 lanes x 16 bytes)

template <bool LR, bool MU>
__global__ __launch_bounds__(256, 1) void w4a4_gemm_dma_kernel(
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, const uint8_t* __restrict__ xcodes,
    const uint8_t* __restrict__ xscales, int M, int N, int K, const __half* __restrict__ T,
    const __half* __restrict__ L2, int r, const __half* __restrict__ mu, const __half* __restrict__ wbar,
    __half* __restrict__ Y) {
  constexpr int BN = Tile256::BN, BM = Tile256::BM, TN = Tile256::TN, TM = Tile256::TM, NS = DMA_STAGES, SB = DMA_STAGE_BYTES;
  constexpr int A_OFF = 0, B_OFF = BN * 64;                       // within a code stage
  constexpr int SA_OFF = 0, SBM_OFF = BN * 16;                    // within a scale group
  __shared__ __align__(16) uint8_t lds[DMA_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int l32 = lane & 31, h = lane >> 5;

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

  const int KB = K >> 1, KS = K >> 5, nk = K >> 7;
  const v4i rA = rsrc_words(wcodes + (int64_t)n0 * KB, (int64_t)(N - n0) * KB);
  const v4i rB = rsrc_words(xcodes + (int64_t)m0 * KB, (int64_t)(M - m0) * KB);
  const v4i rAS = rsrc_words(wscales + (int64_t)n0 * KS, (int64_t)(N - n0) * KS);
  const v4i rBS = rsrc_words(xscales + (int64_t)m0 * KS, (int64_t)(M - m0) * KS);
  // low-rank operands: L2 rows go with the weight rows (A side), T rows with the tokens
  const v4i rL = rsrc_words(L2 + (int64_t)n0 * r, LR ? (int64_t)(N - n0) * r * 2 : 0);
  const v4i rT = rsrc_words(T + (int64_t)m0 * r, LR ? (int64_t)(M - m0) * r * 2 : 0);

  // wave w fills code rows 64 w .. 64 w + 63 of both operands (four instructions each)
  // and the scale groups of rows 64 w + lane.  Instruction q covers rows 64 w + 16 q ..
  // + 15; the chunk swizzle depends on row bits 1..3 only, so the four instructions share
  // the lane's chunk and differ by 16 rows (a uniform offset).
  const int lrow = 64 * wid + (lane >> 2);
  const int og0 = lrow * KB + 16 * ((lane & 3) ^ chunk_swz(lrow));
  const int osc = (64 * wid + lane) * KS;
  const uint32_t lds0 = lds_addr(lds);
  auto code_load = [&](int ks, int g) {     // code load g (0..7) of k-step ks into stage ks % NS
    const uint32_t st = lds0 + (uint32_t)((ks % NS) * SB);
    const int off = ks < nk ? og0 + (16 * (g & 3) * KB + 64 * ks) : KQ_OOB;
    if (g < 4) lds_load16(rA, st + A_OFF + (64 * wid + 16 * g) * 64, off);
    else lds_load16(rB, st + B_OFF + (64 * wid + 16 * (g - 4)) * 64, off);
  };
  // scale group grp (k-steps 4 grp .. 4 grp + 3), issued only when skip is zero: 16 bytes
  // per row.  When K is not a multiple of 512 the last group's piece runs into the next
  // row's scales (or, on the last row, past the end of the range, which reads zeros per
  // dword); the bytes of k-steps past the last are never read.  The skip is a branch
  // inside the assembly so that the loop body stays one block for the instruction
  // scheduler (a compiler branch here lets it move MFMAs across the barrier).
  auto scale_loads = [&](int grp, int skip) {
    const uint32_t sc = lds0 + (uint32_t)(DMA_SC_OFF + (grp & 1) * DMA_SC_BYTES + 16 * 64 * wid);
    const int off = 4 * grp < nk ? osc + 16 * grp : KQ_OOB;
    asm volatile(
        "s_cmp_lg_u32 %0, 0\n\t"
        "s_cbranch_scc1 1f\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %3, %4, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "buffer_load_dwordx4 %3, %5, 0 offen lds\n"
        "1:"
        :: "s"(__builtin_amdgcn_readfirstlane(skip)), "s"(__builtin_amdgcn_readfirstlane(sc + SA_OFF)),
           "s"(__builtin_amdgcn_readfirstlane(sc + SBM_OFF)), "v"(off), "s"(rAS), "s"(rBS)
        : "memory", "m0", "scc");
  };

  const int wrow_a = wn * 128, wrow_b = wm * 128;
  // Fragment i of a wave reads row wrow + 32 i + l32; the chunk swizzle depends on row bits
  // 1..3 only, so it is the same for every i and the four reads of an operand differ by a
  // constant 2 KiB.
  const int sw = chunk_swz(l32);
  const int fa_base[2] = {A_OFF + (wrow_a + l32) * 64 + 16 * (h ^ sw), A_OFF + (wrow_a + l32) * 64 + 16 * ((2 + h) ^ sw)};
  const int fb_base[2] = {B_OFF + (wrow_b + l32) * 64 + 16 * (h ^ sw), B_OFF + (wrow_b + l32) * 64 + 16 * ((2 + h) ^ sw)};
  auto read_frags = [&](const uint8_t* base, int sl, v8i* fa, v8i* fb) {
#pragma unroll
    for (int i = 0; i < TN; ++i) fa[i] = fp4_operand(*reinterpret_cast<const v4i*>(base + fa_base[sl] + 2048 * i));
#pragma unroll
    for (int j = 0; j < TM; ++j) fb[j] = fp4_operand(*reinterpret_cast<const v4i*>(base + fb_base[sl] + 2048 * j));
  };
  const int sa_base = SA_OFF + 16 * (wrow_a + l32), sb_base = SBM_OFF + 16 * (wrow_b + l32);
  auto read_scales = [&](int ks, int* sa, int* sb) {   // the scale dwords of k-step ks
    const uint8_t* sc = lds + DMA_SC_OFF + ((ks >> 2) & 1) * DMA_SC_BYTES + 4 * (ks & 3);
#pragma unroll
    for (int i = 0; i < TN; ++i) sa[i] = (int)(*reinterpret_cast<const uint32_t*>(sc + sa_base + 512 * i) >> (8 * h));
#pragma unroll
    for (int j = 0; j < TM; ++j) sb[j] = (int)(*reinterpret_cast<const uint32_t*>(sc + sb_base + 512 * j) >> (8 * h));
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Prologue: scale group 0 and code stages 0..2, behind the first 32 columns of the
  // low-rank operands, which borrow code stage 3 (16-byte pieces in the same swizzled
  // 64-byte rows as the codes; pieces past column r read as zeros).  The low-rank product
  // enters the accumulators first; r = 64 takes a second pass through the same stage.
  auto lr_load = [&](int rc) {
    const uint32_t st = lds0 + (uint32_t)((NS - 1) * SB);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 64 * wid + 16 * q + (lane >> 2);
      const int piece = 8 * ((lane & 3) ^ chunk_swz(row));     // column of the piece
      const int off = rc + piece < r ? (row * r + rc + piece) * 2 : KQ_OOB;
      lds_load16(rL, st + A_OFF + (64 * wid + 16 * q) * 64, off);
      lds_load16(rT, st + B_OFF + (64 * wid + 16 * q) * 64, off);
    }
  };
  auto lr_mfma = [&]() {
    const uint8_t* base = lds + (NS - 1) * SB;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      v8h lt[TM], ll[TN];
      const int ch = 2 * c2 + h;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int row = wrow_a + 32 * i + l32;
        ll[i] = *reinterpret_cast<const v8h*>(base + A_OFF + row * 64 + 16 * (ch ^ chunk_swz(row)));
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int row = wrow_b + 32 * j + l32;
        lt[j] = *reinterpret_cast<const v8h*>(base + B_OFF + row * 64 + 16 * (ch ^ chunk_swz(row)));
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ll[i], lt[j], acc[i][j], 0, 0, 0);
    }
  };
  // Rank-1 restore operands.  The token means of this lane's four rows go straight into
  // registers (rows past M repeat the last mean; they are never stored).  They are the
  // oldest loads of the wave, so the k-loop's counted waits cover them.  The tile's 256
  // column sums go to LDS with one 16-byte load per lane of lanes 0..31 (the others read
  // past the range and write zeros): N is a multiple of 16, so a piece is wholly inside
  // or wholly outside the row of sums, never cut by the range check.
  float mu_r[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) mu_r[j] = 0.0f;
  if (MU) {
#pragma unroll
    for (int j = 0; j < TM; ++j) mu_r[j] = __half2float(mu[min(m0 + wm * 128 + 32 * j + l32, M - 1)]);
  }
  if (MU && wid == 0) {
    const v4i rW = rsrc_words(wbar + n0, (int64_t)(N - n0) * 2);
    const int off = lane < 32 ? 16 * lane : KQ_OOB;
    lds_load16(rW, lds0 + DMA_MU_OFF, off);
  }
  if (LR) lr_load(0);
  scale_loads(0, 0);
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
#pragma unroll
    for (int g = 0; g < DMA_CODE_LOADS; ++g) code_load(p, g);
  if (LR) {
    // the low-rank pieces and everything before the 16 youngest loads (scale group 0,
    // code stage 0) have landed once at most 16 loads of this wave are outstanding
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * DMA_CODE_LOADS));
    lds_barrier();
    lr_mfma();
    for (int rc = 32; rc < r; rc += 32) {
      lds_barrier();                              // every wave has read the previous chunk
      lr_load(rc);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
      lr_mfma();
    }
    lds_barrier();                                // stage 3 is free for the k-loop's loads
  }

  // k-loop.  The loads of k-steps past the last one write zeros into stages that are
  // never computed; they are drained before the epilogue.  Per k-step:
  //   slice-0 MFMAs, interleaved with the slice-1 fragment reads of ks and the first four
  //     code loads of ks + 3 (the address unit is shared by the workgroup's four waves:
  //     issued in a burst, the loads would stall the wave -- and its matrix core -- for
  //     their whole issue time);
  //   wait for this wave's loads of ks + 1, barrier;
  //   at the start of a group of four k-steps, the next group's scale loads;
  //   slice-1 MFMAs, interleaved with the scale and slice-0 fragment reads of ks + 1 and
  //     the last four code loads of ks + 3.
  if (!LR) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * DMA_CODE_LOADS));
    lds_barrier();
  }
  v8i a0[TN], b0[TM];
  int sa[TN], sb[TM];
  read_scales(0, sa, sb);
  read_frags(lds, 0, a0, b0);
  for (int ks = 0; ks < nk; ++ks) {
    const uint8_t* const cur = lds + (ks % NS) * SB;
    const uint8_t* const nxt = lds + ((ks + 1) % NS) * SB;
    v8i a1[TN], b1[TM];
    __builtin_amdgcn_sched_barrier(0);
    // slice 0: MFMA m is preceded by slice-1 fragment m (m < 8: four A, then four B) and
    // followed, for m = 1, 5, 9, 13, by code load (m - 1) / 4 of k-step ks + 3
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = TM * i + j;
        if (m < 8) {
          __builtin_amdgcn_sched_barrier(0);
          if (m < 4) a1[m] = fp4_operand(*reinterpret_cast<const v4i*>(cur + fa_base[1] + 2048 * m));
          else b1[m - 4] = fp4_operand(*reinterpret_cast<const v4i*>(cur + fb_base[1] + 2048 * (m - 4)));
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0[i], b0[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
        if (m % 4 == 1) {
          __builtin_amdgcn_sched_barrier(0);
          code_load(ks + NS - 1, m / 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // k-step ks + 1 has landed once at most 12 of this wave's loads are outstanding: those
    // of ks + 2 and the first half of ks + 3 (the second half of ks + 1 went out before
    // any of them)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * DMA_CODE_LOADS - DMA_CODE_LOADS / 2));
    lds_barrier();
    scale_loads((ks >> 2) + 1, ks & 3);
    int nsa[TN], nsb[TM];
    const uint8_t* const sc = lds + DMA_SC_OFF + (((ks + 1) >> 2) & 1) * DMA_SC_BYTES + 4 * ((ks + 1) & 3);
    __builtin_amdgcn_sched_barrier(0);
    // slice 1: MFMA m is followed by read m of the next k-step (four A scales, four B
    // scales, four A fragments, four B fragments of slice 0) and, for m = 1, 5, 9, 13, by
    // code load 4 + (m - 1) / 4 of k-step ks + 3 (its stage was freed by the barrier above)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = TM * i + j;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[i], b1[j], acc[i][j], 4, 4, 2, sa[i], 2, sb[j]);
        __builtin_amdgcn_sched_barrier(0);
        if (m < 4) nsa[m] = (int)(*reinterpret_cast<const uint32_t*>(sc + sa_base + 512 * m) >> (8 * h));
        else if (m < 8) nsb[m - 4] = (int)(*reinterpret_cast<const uint32_t*>(sc + sb_base + 512 * (m - 4)) >> (8 * h));
        else if (m < 12) a0[m - 8] = fp4_operand(*reinterpret_cast<const v4i*>(nxt + fa_base[0] + 2048 * (m - 8)));
        else b0[m - 12] = fp4_operand(*reinterpret_cast<const v4i*>(nxt + fb_base[0] + 2048 * (m - 12)));
        __builtin_amdgcn_sched_barrier(0);
        if (m % 4 == 1) {
          code_load(ks + NS - 1, 4 + m / 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
    for (int i = 0; i < TN; ++i) sa[i] = nsa[i];
#pragma unroll
    for (int j = 0; j < TM; ++j) sb[j] = nsb[j];
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no load may land in LDS after the workgroup ends

  const __amdgpu_buffer_rsrc_t rY = make_rsrc(Y + (int64_t)m0 * N, (int64_t)(M - m0) * N * 2);
  const __half* const wbar_t = reinterpret_cast<const __half*>(lds + DMA_MU_OFF);
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int ml = wrow_b + 32 * j + l32;
    const float mm = mu_r[j];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t pk[2][2];                                   // [group of the pair][dword]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int g = 2 * p + u;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
          if (MU) {
            // halves unpacked from scalar dwords (a bit cast of a vector element inside an
            // unrolled loop is mis-compiled to read element 0)
            const uint32_t* const wp = reinterpret_cast<const uint32_t*>(wbar_t + wrow_a + 32 * i + 8 * g + 4 * h);
            const uint32_t w01 = wp[0], w23 = wp[1];
            v[0] = __builtin_fmaf(mm, __half2float(__ushort_as_half((unsigned short)(w01 & 0xFFFFu))), v[0]);
            v[1] = __builtin_fmaf(mm, __half2float(__ushort_as_half((unsigned short)(w01 >> 16))), v[1]);
            v[2] = __builtin_fmaf(mm, __half2float(__ushort_as_half((unsigned short)(w23 & 0xFFFFu))), v[2]);
            v[3] = __builtin_fmaf(mm, __half2float(__ushort_as_half((unsigned short)(w23 >> 16))), v[3]);
          }
          pk[u][0] = __builtin_bit_cast(uint32_t, __floats2half2_rn(v[0], v[1]));
          pk[u][1] = __builtin_bit_cast(uint32_t, __floats2half2_rn(v[2], v[3]));
        }
        // a lane holds columns 8 g + 4 h .. + 3 of groups g = 2p, 2p + 1; one lane-half swap
        // per dword leaves lanes 0..31 with the eight columns of group 2p and lanes 32..63
        // with those of group 2p + 1: one 16-byte store per lane
        const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
        const v4u outv = {s0[0], s1[0], s0[1], s1[1]};
        const int col = wrow_a + 32 * i + 8 * (2 * p + h);
        const int off = n0 + col < N ? (ml * N + n0 + col) * 2 : KQ_OOB;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, outv), rY, off, 0, 0);
      }
    }
  }
}

static hipError_t gemm_dma_launch(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                                 const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                                 const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                                 hipStream_t s) {
  const int64_t tiles = ((N + Tile256::BN - 1) / Tile256::BN) * ((M + Tile256::BM - 1) / Tile256::BM);
  const dim3 g((unsigned)tiles), b(Tile256::NT);
  if (r > 0 && mu)
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<true, true>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  else if (r > 0)
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<true, false>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  else if (mu)
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<false, true>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  else
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<false, false>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y);
  return hipGetLastError();
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

hipError_t launch_w4a4_gemm(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                            const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                            hipStream_t s) {
  // K is a multiple of 128 (the entry points check it): above a quarter round of 256 x 256
  // tiles the direct-to-LDS form, at or below it 128 x 128 tiles staged through registers
  // (measured: the large tiles win from 72 of them up, by up to 11% at 96; the small ones
  // at 64 and below, by up to 25% at 40)
  using Small = GemmCfg<128, 128, 2, 2, 1>;
  const int64_t big_tiles = ((N + 255) / 256) * ((M + 255) / 256);
  if (4 * big_tiles > device_cu_count())
    return gemm_dma_launch(xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, s);
  return gemm_launch<Small>(xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, s);
}

}  // namespace kq
