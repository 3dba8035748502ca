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
// lane ends with four consecutive output columns of one output row.
//
// One kernel: tiles of 256 token rows by 256 weight rows (or 128 in the last round of a
// grid), their operands going from global memory straight into LDS (buffer loads with the
// LDS destination), four stages deep.  Per 128-wide k-step a row contributes 64 code bytes
// and 4 scale bytes.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row, so that the 16-byte
// MFMA fragment reads (16 rows x one chunk) and the staging writes hit distinct banks.
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// The rank-1 FMA's fp32 results, hidden from the compiler (an empty statement that takes and
// returns the registers), so that every output rounds twice, to fp32 in the FMA and to fp16
// in the conversion: left alone, the compiler fuses some FMAs with the conversion into one
// mixed-precision FMA (one rounding), a different subset for each tile width.
__device__ __forceinline__ void keep_f32(float (&v)[4]) {
  asm("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

// The 32x32x64 form of the scaled FP4 MFMA is the one that runs at the doubled FP4 rate
// on gfx950 (the 16x16x128 form issues at the FP8 rate).  Its operand layout: lane l
// holds row l%32 and k-block l/32 of the 64-wide k-slice (16 bytes = 32 codes) plus that
// block's E8M0 byte; the 32x32 result sits in 16 registers, register 4g+i of lane l being
// C[8g + 4(l/32) + i][l%32].
//
// 256x256 tiles on 4 wavefronts (2 x 2), each owning a 128 x 128 block of 4 x 4 MFMA tiles
// (256 fp32 accumulators per lane, held in the accumulation registers), which halves the
// LDS bytes read per MFMA against 128 x 64 wave tiles.  Per 128-wide
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

// One output tile: 64 TN weight rows from n0 by 256 token rows from m0.  TN = 4 is the
// 256 x 256 tile; TN = 2 a tile of half its width (wavefront tiles of 64 x 128), for the
// last tile rows of a grid whose last round would otherwise be partly empty.  Both use
// the full tile's LDS layout; the half tile leaves weight rows 128 .. 255 of each code
// stage unused (its scale, low-rank and column-sum staging still fills them, unread).
template <bool LR, bool MU, int TN>
__device__ __forceinline__ void dma_tile(uint8_t* __restrict__ lds, const uint8_t* __restrict__ wcodes,
                                         const uint8_t* __restrict__ wscales, const uint8_t* __restrict__ xcodes,
                                         const uint8_t* __restrict__ xscales, int M, int N, int K,
                                         const __half* __restrict__ T, const __half* __restrict__ L2, int r,
                                         const __half* __restrict__ mu, const __half* __restrict__ wbar,
                                         __half* __restrict__ Y, int m0, int n0) {
  constexpr int BN = Tile256::BN, TM = Tile256::TM, NS = DMA_STAGES, SB = DMA_STAGE_BYTES;
  constexpr int NL = TN == 4 ? DMA_CODE_LOADS : 6;   // code loads per wave and k-step
  constexpr int NA = TN == 4 ? 4 : 2;                // of which weight rows (16 rows each)
  constexpr int A_OFF = 0, B_OFF = BN * 64;                       // within a code stage
  constexpr int SA_OFF = 0, SBM_OFF = BN * 16;                    // within a scale group
  // the thread index, hidden from the compiler: in the kernel's tile loop it would otherwise
  // hoist every lane-dependent offset out of the loop and keep them live through it (spilling)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int l32 = lane & 31, h = lane >> 5;

  const int KB = K >> 1, KS = K >> 5, nk = K >> 7;
  const v4i rA = rsrc_words(wcodes + (int64_t)n0 * KB, (int64_t)(N - n0) * KB);
  const v4i rB = rsrc_words(xcodes + (int64_t)m0 * KB, (int64_t)(M - m0) * KB);
  const v4i rAS = rsrc_words(wscales + (int64_t)n0 * KS, (int64_t)(N - n0) * KS);
  const v4i rBS = rsrc_words(xscales + (int64_t)m0 * KS, (int64_t)(M - m0) * KS);
  // low-rank operands: L2 rows go with the weight rows (A side), T rows with the tokens
  const v4i rL = rsrc_words(L2 + (int64_t)n0 * r, LR ? (int64_t)(N - n0) * r * 2 : 0);
  const v4i rT = rsrc_words(T + (int64_t)m0 * r, LR ? (int64_t)(M - m0) * r * 2 : 0);

  // wave w fills token rows 64 w .. 64 w + 63 (four instructions) and weight rows
  // 16 NA w .. 16 NA (w + 1) - 1 (NA instructions), and the scale groups of rows 64 w + lane
  // of both operands.  An instruction covers 16 rows; the chunk swizzle depends on row
  // bits 1..3 only, so all of a wave's instructions share the lane's chunk and differ by
  // multiples of 16 rows (uniform offsets).
  const int csw = 16 * ((lane & 3) ^ chunk_swz(lane >> 2));
  const int ogA = (16 * NA * wid + (lane >> 2)) * KB + csw;
  const int ogB = (64 * wid + (lane >> 2)) * KB + csw;
  const int osc = (64 * wid + lane) * KS;
  const uint32_t lds0 = lds_addr(lds);
  auto code_load = [&](int ks, int g) {     // code load g (0 .. NL - 1) of k-step ks into stage ks % NS
    const uint32_t st = lds0 + (uint32_t)((ks % NS) * SB);
    if (g < NA) {
      const int off = ks < nk ? ogA + (16 * g * KB + 64 * ks) : KQ_OOB;
      lds_load16(rA, st + A_OFF + (16 * NA * wid + 16 * g) * 64, off);
    } else {
      const int off = ks < nk ? ogB + (16 * (g - NA) * KB + 64 * ks) : KQ_OOB;
      lds_load16(rB, st + B_OFF + (64 * wid + 16 * (g - NA)) * 64, off);
    }
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

  const int wrow_a = wn * 32 * TN, wrow_b = wm * 128;
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
    for (int g = 0; g < NL; ++g) code_load(p, g);
  if (LR) {
    // the low-rank pieces and everything before the 16 youngest loads (scale group 0,
    // code stage 0) have landed once at most 16 loads of this wave are outstanding
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * NL));
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
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * NL));
    lds_barrier();
  }
  constexpr int NM = TN * TM;            // MFMAs per slice
  constexpr int LST = NM / (NL / 2);     // MFMAs between code loads
  constexpr int NR = 2 * (TN + TM);      // reads of the next k-step during slice 1
  v8i a0[TN], b0[TM];
  int sa[TN], sb[TM];
  read_scales(0, sa, sb);
  read_frags(lds, 0, a0, b0);
  for (int ks = 0; ks < nk; ++ks) {
    const uint8_t* const cur = lds + (ks % NS) * SB;
    const uint8_t* const nxt = lds + ((ks + 1) % NS) * SB;
    v8i a1[TN], b1[TM];
    __builtin_amdgcn_sched_barrier(0);
    // slice 0: MFMA m is preceded by slice-1 fragment m (m < TN + TM: the A ones, then
    // the B ones) and followed, for m = 1, 1 + LST, 1 + 2 LST, .., by the first NL / 2 code
    // loads of k-step ks + 3
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = TM * i + j;
        if (m < TN + TM) {
          __builtin_amdgcn_sched_barrier(0);
          if (m < TN) a1[m] = fp4_operand(*reinterpret_cast<const v4i*>(cur + fa_base[1] + 2048 * m));
          else b1[m - TN] = fp4_operand(*reinterpret_cast<const v4i*>(cur + fb_base[1] + 2048 * (m - TN)));
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0[i], b0[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
        if (m % LST == 1 && m / LST < NL / 2) {
          __builtin_amdgcn_sched_barrier(0);
          code_load(ks + NS - 1, m / LST);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // k-step ks + 1 has landed once at most 3 NL / 2 of this wave's loads are
    // outstanding: those of ks + 2 and the first half of ks + 3 (the second half of ks + 1
    // went out before any of them)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * NL - NL / 2));
    lds_barrier();
    scale_loads((ks >> 2) + 1, ks & 3);
    int nsa[TN], nsb[TM];
    const uint8_t* const sc = lds + DMA_SC_OFF + (((ks + 1) >> 2) & 1) * DMA_SC_BYTES + 4 * ((ks + 1) & 3);
    __builtin_amdgcn_sched_barrier(0);
    // slice 1: MFMA m is followed by reads NR m / NM .. NR (m + 1) / NM - 1 of the next
    // k-step (TN A scales, TM B scales, then the slice-0 fragments: TN A, TM B) and, for
    // m = 1, 1 + LST, .., by the last NL / 2 code loads of k-step ks + 3 (their stage was
    // freed by the barrier above)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = TM * i + j;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1[i], b1[j], acc[i][j], 4, 4, 2, sa[i], 2, sb[j]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = NR * m / NM; q < NR * (m + 1) / NM; ++q) {
          if (q < TN) nsa[q] = (int)(*reinterpret_cast<const uint32_t*>(sc + sa_base + 512 * q) >> (8 * h));
          else if (q < TN + TM)
            nsb[q - TN] = (int)(*reinterpret_cast<const uint32_t*>(sc + sb_base + 512 * (q - TN)) >> (8 * h));
          else if (q < 2 * TN + TM)
            a0[q - TN - TM] = fp4_operand(*reinterpret_cast<const v4i*>(nxt + fa_base[0] + 2048 * (q - TN - TM)));
          else
            b0[q - 2 * TN - TM] = fp4_operand(*reinterpret_cast<const v4i*>(nxt + fb_base[0] + 2048 * (q - 2 * TN - TM)));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (m % LST == 1 && m / LST < NL / 2) {
          code_load(ks + NS - 1, NL / 2 + m / LST);
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
            keep_f32(v);
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

// The direct-to-LDS form's kernel.  The first full_rows rows of 256 x 256 tiles take the
// full tile, grouped eight tile rows at a time along M (column-major within a group) for
// L2 reuse; the tile rows below them, if any, take tiles of half the width, one per
// workgroup.  With no half-width tiles, each workgroup loops over every grid-th tile.
// Within each part, consecutive tile numbers (which the dispatcher deals out to the compute
// dies in turn) are remapped so that each die holds a contiguous run of tiles.
template <bool LR, bool MU>
__global__ __launch_bounds__(256, 1) void w4a4_gemm_dma_kernel(
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, const uint8_t* __restrict__ xcodes,
    const uint8_t* __restrict__ xscales, int M, int N, int K, const __half* __restrict__ T,
    const __half* __restrict__ L2, int r, const __half* __restrict__ mu, const __half* __restrict__ wbar,
    __half* __restrict__ Y, int full_rows) {
  __shared__ __align__(16) uint8_t lds[DMA_LDS];
  const int tiles_n = (N + 255) / 256;
  const int nfull = tiles_n * full_rows;
  auto full_tile = [&](int pid) {
    {
      const int per = nfull / 8;
      if (pid < 8 * per) pid = (pid % 8) * per + pid / 8;
    }
    constexpr int GM = 8;
    const int group = pid / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsize = min(full_rows - first_m, GM);
    const int tile_m = first_m + (pid % (GM * tiles_n)) % gsize;
    const int tile_n = (pid % (GM * tiles_n)) / gsize;
    dma_tile<LR, MU, 4>(lds, wcodes, wscales, xcodes, xscales, M, N, K, T, L2, r, mu, wbar, Y, 256 * tile_m,
                        256 * tile_n);
  };
  if (full_rows == (M + 255) / 256) {
    // full tiles only: workgroup b takes tiles b, b + G, .. (G = the grid, a multiple of the 8
    // compute dies, so a tile stays on the die the remap assumes); the barrier keeps the next
    // tile's staging loads off the column sums this tile's epilogue still reads
    for (int t = blockIdx.x; t < nfull; t += gridDim.x) {
      full_tile(t);
      __syncthreads();
    }
    return;
  }
  const int pid = blockIdx.x;
  if (pid < nfull) {
    full_tile(pid);
  } else {
    const int hrows = (M + 255) / 256 - full_rows;
    const int nh = ((N + 127) / 128) * hrows;
    int q = pid - nfull;
    {
      const int per = nh / 8;
      if (q < 8 * per) q = (q % 8) * per + q / 8;
    }
    const int tile_m = full_rows + q % hrows, tile_n = q / hrows;
    dma_tile<LR, MU, 2>(lds, wcodes, wscales, xcodes, xscales, M, N, K, T, L2, r, mu, wbar, Y, 256 * tile_m,
                        128 * tile_n);
  }
}

static hipError_t gemm_dma_launch(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                                 const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                                 const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                                 hipStream_t s) {
  // A last round of tiles that leaves compute units idle costs nearly as much as a full
  // one (measured at M = 4608, K = 3072: three rounds 98.8 us, three rounds and 18 tiles
  // 118.6 us).  The last tile rows go to tiles of half the width when those fit in one
  // round: the grid then ends with a round of half-length tiles.
  const int64_t tiles_n = (N + 255) / 256, tiles_m = (M + 255) / 256, tiles_n2 = (N + 127) / 128;
  const int64_t cus = device_cu_count();
  const int64_t ntiles = tiles_n * tiles_m;
  const int64_t tail = ntiles % cus;
  int64_t full_rows = tiles_m;
  if (tail > 0) {
    const int64_t hr = (tail + tiles_n - 1) / tiles_n;     // tile rows that hold the tail
    if (hr * tiles_n2 <= cus) full_rows = tiles_m - hr;
  }
  int64_t grid = tiles_n * full_rows + tiles_n2 * (tiles_m - full_rows);
  if (full_rows == tiles_m) {
    // Otherwise the rounds are made even: as many workgroups as the largest round needs
    // (rounded up to a multiple of the 8 dies), each taking every grid-th tile.  Measured:
    // 1.5 rounds of tiles 4% faster as two rounds of 192, 12.9 rounds 2% faster as a loop
    // over 256 workgroups; 2.5-2.8 rounds unchanged.
    const int64_t rounds = (ntiles + cus - 1) / cus;
    const int64_t even = ((ntiles + rounds - 1) / rounds + 7) / 8 * 8;
    if (even < grid) grid = even;
  }
  const dim3 g((unsigned)grid), b(Tile256::NT);
  if (r > 0 && mu)
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<true, true>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y, (int)full_rows);
  else if (r > 0)
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<true, false>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y, (int)full_rows);
  else if (mu)
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<false, true>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y, (int)full_rows);
  else
    hipLaunchKernelGGL((w4a4_gemm_dma_kernel<false, false>), g, b, 0, s, wcodes, wscales, xcodes, xscales, (int)M,
                       (int)N, (int)K, T, L2, r, mu, wbar, Y, (int)full_rows);
  return hipGetLastError();
}

hipError_t launch_w4a4_gemm(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const uint8_t* wscales, int64_t N, const __half* T,
                            const __half* L2, int r, const __half* mu, const __half* wbar, __half* Y,
                            hipStream_t s) {
  // K is a multiple of 128 (the entry points check it)
  return gemm_dma_launch(xcodes, xscales, M, K, wcodes, wscales, N, T, L2, r, mu, wbar, Y, s);
}

}  // namespace kq
