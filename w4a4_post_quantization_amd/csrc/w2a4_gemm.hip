// W2A4 linear for the rotated, calibration-free path (OrbitQuant §03: one Lloyd-Max
// codebook for all rotated coordinates; §04: 2-bit weights, 4-bit activations; CentriQ
// abstract: closed-form per-token scale):
//   Y[m][n] = s_t[m] * sum_g s_g[n][g] * sum_{k in g} l16[qx[m][k]] * l4[qw[n][k]].
// The codes are dequantized to fp16 in registers (byte-permute table lookups: activation
// levels without their per-token scale, weight levels times their fp16 group scale), staged
// in LDS once per workgroup tile and multiplied on the fp16 matrix cores (fp32
// accumulation); the per-token scale multiplies the accumulator before the fp16 store.  Two
// forms: 128 x 128 tiles of 16 x 16 x 32 products for small grids, and 256 x 256 tiles (or
// 256 x 128 ones in a grid's last round) of 32 x 32 x 16 products.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int chunk_swz2(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Dequantization in registers, by byte permutes (v_perm_b32 picks each result byte out of
// eight source bytes, so two registers form an eight-entry byte table):
//   - activation codes (4 bits, bit 3 the sign): the low and the high bytes of the eight
//     fp16 magnitude levels are two such tables; the sign goes into bit 15;
//   - weight codes (2 bits, bit 1 the sign): the low and the high bytes of the group's four
//     fp16 values (both magnitudes times the group scale, and their negations) are two
//     four-entry tables indexed by the code.
// The values are the same fp16 numbers a table of fp16(+-level) (times the scale, one
// fp16 product) would hold: negation only flips the sign bit.
struct LmRegTables {
  uint32_t lo0, lo1, hi0, hi1;   // bytes of fp16(l16[m]): low bytes m = 0..3, 4..7, then high bytes
  uint32_t l4;                   // fp16(l4[0]) | fp16(l4[1]) << 16
};

__device__ __forceinline__ LmRegTables lm_reg_tables(const LmTables& lm) {
  LmRegTables t{0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t hv = __half_as_ushort(__float2half_rn(lm.l16[m]));
    const int sh = 8 * (m & 3);
    if (m < 4) {
      t.lo0 |= (hv & 0xFFu) << sh;
      t.hi0 |= (hv >> 8) << sh;
    } else {
      t.lo1 |= (hv & 0xFFu) << sh;
      t.hi1 |= (hv >> 8) << sh;
    }
  }
  t.l4 = __builtin_bit_cast(uint32_t, __floats2half2_rn(lm.l4[0], lm.l4[1]));
  return t;
}

// Both operands' eight values of an 8-code chunk are produced in the order
// (0, 4, 1, 5, 2, 6, 3, 7) of their k positions, the order in which the permutes deliver
// them most cheaply; the A and B chunks share it, so every product pairs the same k.

// Eight 4-bit activation codes (code i in bits 4i .. 4i + 3) -> eight fp16 levels, two per
// dword: (0, 4), (1, 5), (2, 6), (3, 7).
__device__ __forceinline__ void dequant_a4(uint32_t x, const LmRegTables& t, uint32_t out[4]) {
  const uint32_t me = x & 0x07070707u, mo = (x >> 4) & 0x07070707u;   // magnitudes: codes 0,2,4,6 / 1,3,5,7
  const uint32_t le = __builtin_amdgcn_perm(t.lo1, t.lo0, me);
  const uint32_t he = __builtin_amdgcn_perm(t.hi1, t.hi0, me) | ((x & 0x08080808u) << 4);
  const uint32_t lo = __builtin_amdgcn_perm(t.lo1, t.lo0, mo);
  const uint32_t ho = __builtin_amdgcn_perm(t.hi1, t.hi0, mo) | (x & 0x80808080u);
  out[0] = __builtin_amdgcn_perm(he, le, 0x06020400u);   // codes 0, 4
  out[1] = __builtin_amdgcn_perm(ho, lo, 0x06020400u);   // codes 1, 5
  out[2] = __builtin_amdgcn_perm(he, le, 0x07030501u);   // codes 2, 6
  out[3] = __builtin_amdgcn_perm(ho, lo, 0x07030501u);   // codes 3, 7
}

// The group's tables for weight codes: the low and the high bytes of (+m0, +m1, -m0, -m1),
// m = fp16(l4) * fp16 scale (one fp16 product each).
__device__ __forceinline__ void w2_group_table(const LmRegTables& t, __half sg, uint32_t& tlo, uint32_t& thi) {
  const uint32_t m = __builtin_bit_cast(uint32_t, __hmul2(__builtin_bit_cast(__half2, t.l4), __half2half2(sg)));
  tlo = __builtin_amdgcn_perm(m, m, 0x02000200u);
  thi = __builtin_amdgcn_perm(m, m, 0x03010301u) ^ 0x80800000u;
}

// Eight 2-bit weight codes (code i in bits 2i, 2i + 1 of x, x < 2^16) -> eight fp16 values in
// the same order.  With z = x | x << 14, the bytes of z & 0x03030303 are codes 0, 4, 1, 5 and
// those of (z >> 4) & 0x03030303 codes 2, 6, 3, 7: each byte selects its value's low and
// high byte from the group's tables.
__device__ __forceinline__ void dequant_w2(uint32_t x, uint32_t tlo, uint32_t thi, uint32_t out[4]) {
  const uint32_t z = x | (x << 14);
  const uint32_t s1 = z & 0x03030303u, s2 = (z >> 4) & 0x03030303u;
  const uint32_t l1 = __builtin_amdgcn_perm(0u, tlo, s1), h1 = __builtin_amdgcn_perm(0u, thi, s1);
  const uint32_t l2 = __builtin_amdgcn_perm(0u, tlo, s2), h2 = __builtin_amdgcn_perm(0u, thi, s2);
  out[0] = __builtin_amdgcn_perm(h1, l1, 0x05010400u);   // codes 0, 4
  out[1] = __builtin_amdgcn_perm(h1, l1, 0x07030602u);   // codes 1, 5
  out[2] = __builtin_amdgcn_perm(h2, l2, 0x05010400u);   // codes 2, 6
  out[3] = __builtin_amdgcn_perm(h2, l2, 0x07030602u);   // codes 3, 7
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

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid % WN, wm = wid / WN;
  const int lr = lane & 15, q = lane >> 4;
  const LmRegTables lt = lm_reg_tables(lm);

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
      uint32_t t0, t1;
      w2_group_table(lt, sg, t0, t1);
      const uint32_t wv[2] = {raw.x, raw.y};
#pragma unroll
      for (int c = 0; c < 4; ++c) dequant_w2((wv[c >> 1] >> (16 * (c & 1))) & 0xFFFFu, t0, t1, h + 4 * c);
    } else {
      const uint32_t xv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) dequant_a4(xv[c], lt, h + 4 * c);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint4*>(base + 16 * (c ^ sw)) = make_uint4(h[4 * c], h[4 * c + 1], h[4 * c + 2], h[4 * c + 3]);
  };

  const int wrow_a = wn * (BN / WN), wrow_b = wm * (BM / WM);
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

// Large-tile form: 64 TN weight rows (TN = 4: 256; TN = 2: 128, a tile of half the width
// for the last round of a grid) x 256 tokens per workgroup on 4 wavefronts (2 x 2), each
// owning a 32 TN x 128 block of 32 x 32 output tiles (v_mfma_f32_32x32x16_f16: lane l
// holds row l % 32 and k = 8 (l / 32) .. + 7 of each 16-wide step; result register 4 g + e
// of lane l is C[8 g + 4 (l / 32) + e][l % 32]).  Against 64 x 64 wave tiles of 16 x 16
// products the full tile reads half the LDS bytes per product.  A k-step is two groups
// (64 k) held as fp16 in one of two LDS buffers: thread t dequantizes token row t and
// weight row t (TN = 4) or one group of weight row t / 2 (TN = 2) into the buffer the next
// step reads, LDS rows of 128 bytes with their 16-byte chunks XOR-swizzled by the row's low
// bits.  Schedule of a step, pinned with scheduling barriers so that the matrix cores never
// wait for a whole phase:
//   - the fragments of the step's first 16-wide slice are read;
//   - the 16 TN products run as four slices of 4 TN; after each of the first TN + 4
//     products of a slice one fragment of the next slice is read, and the thread's 8-code
//     chunks of the next step (16, or 12 in the half-width tile) are dequantized and stored
//     to the other buffer one at a time, spread evenly over the products;
//   - one barrier: the next step's buffer is complete, this one is free.
// The codes a step dequantizes were loaded one step earlier (the loads of step ks + 2 go
// out during step ks, one at a time between products), so the dequantization never waits
// for memory.  Loads past the last step or of a missing second group (K % 64 = 32) are
// outside the buffer ranges and read zeros: the group's scale is then zero and so are its
// products.
template <int TN>
struct W2Raw {                     // the codes of one step that a thread stages
  v2u w[TN == 4 ? 2 : 1];          // weight codes: both groups of its row, or its one group
  uint32_t s[TN == 4 ? 2 : 1];     // their fp16 group scales
  v4u x[2];                        // activation codes of both groups of its token row
};

// The chunk dequantized after product p of a step (-1: none): in the full tile after every
// fourth product; in the half-width tile chunk j after product 8 j / 3 + 2.
template <int TN>
__host__ __device__ constexpr int w2_dq_at(int p) {
  if (TN == 4) return (p & 3) == 3 ? p >> 2 : -1;
  for (int j = 0; j < 12; ++j)
    if (p == 8 * j / 3 + 2) return j;
  return -1;
}

// The load issued after product m of slice sub (-1: none): six per step in the full tile
// (weight codes, scale and activation codes of each group), four in the half-width tile
// (its group's weight codes and scale, the two groups' activation codes).
template <int TN>
__host__ __device__ constexpr int w2_load_at(int sub, int m) {
  if (TN == 4) return sub < 3 && (m == 1 || m == 9) ? 2 * sub + (m >> 3) : -1;
  return sub < 2 && (m == 1 || m == 5) ? 2 * sub + (m >> 2) : -1;
}

template <int TN>
__device__ __forceinline__ void w2a4_big_tile(uint8_t* __restrict__ lds, const uint8_t* __restrict__ xcodes,
                                              const float* __restrict__ xscales, int M, int K,
                                              const uint8_t* __restrict__ wcodes, const __half* __restrict__ wscales,
                                              int N, const LmRegTables& lt, __half* __restrict__ Y, int m0, int n0) {
  constexpr int TM = 4, RB = 128;                       // RB: LDS bytes per row and step
  constexpr int A_OFF = 0, B_OFF = 256 * RB, BUF = 512 * RB;   // the full tile's layout in both widths
  constexpr int NWC = TN == 4 ? 8 : 4;                  // weight chunks a thread dequantizes per step
  constexpr int NU = TN == 4 ? 6 : 4;                   // loads a thread issues per step
  // the thread index, hidden from the compiler: in the kernel's tile loop it would otherwise
  // hoist every lane-dependent offset out of the loop and keep them live through it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int ng = K >> 5, nks = (ng + 1) >> 1;             // groups, 64-wide steps

  // staging rows of this thread, relative to the tile: token row tid, and weight row tid
  // (both groups of a step) or weight row tid / 2 (group tid % 2 of a step); rows past the
  // matrix repeat its last row (their results are never stored)
  const int wrow = TN == 4 ? tid : tid >> 1, wq = TN == 4 ? 0 : tid & 1;
  const int wr = min(n0 + wrow, N - 1) - n0, xr = min(m0 + tid, M - 1) - m0;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(wcodes + (int64_t)n0 * (K >> 2), (int64_t)(N - n0) * (K >> 2));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(wscales + (int64_t)n0 * ng, (int64_t)(N - n0) * ng * 2);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(xcodes + (int64_t)m0 * (K >> 1), (int64_t)(M - m0) * (K >> 1));
  const int ow = wr * (K >> 2), os = wr * ng * 2, ox = xr * (K >> 1);
  const int swa = wrow & 7, swb = tid & 7;

  // load u of step ks.  Each load touches one cache line per lane (a row per thread), so
  // they go out one at a time between products: issued together they would hold the wave,
  // and its matrix core, for their whole address-unit time.
  auto gload1 = [&](int ks, W2Raw<TN>& r, int u) {
    if (TN == 4) {            // u / 3 is the group, u % 3 picks weight codes, scale or activation codes
      const int q = u / 3;
      const bool v = 2 * ks + q < ng;
      if (u % 3 == 0)
        r.w[q] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rW, v ? ow + 16 * ks + 8 * q : KQ_OOB, 0, 0));
      else if (u % 3 == 1)
        r.s[q] = __builtin_amdgcn_raw_buffer_load_b16(rS, v ? os + 4 * ks + 2 * q : KQ_OOB, 0, 0);
      else
        r.x[q] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rX, v ? ox + 32 * ks + 16 * q : KQ_OOB, 0, 0));
    } else if (u < 2) {       // the thread's group of its weight row: codes, then scale
      const bool v = 2 * ks + wq < ng;
      if (u == 0)
        r.w[0] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rW, v ? ow + 16 * ks + 8 * wq : KQ_OOB, 0, 0));
      else
        r.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rS, v ? os + 4 * ks + 2 * wq : KQ_OOB, 0, 0);
    } else {                  // activation codes of group u - 2
      const int q = u - 2;
      const bool v = 2 * ks + q < ng;
      r.x[q] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rX, v ? ox + 32 * ks + 16 * q : KQ_OOB, 0, 0));
    }
  };
  auto gload = [&](int ks, W2Raw<TN>& r) {
#pragma unroll
    for (int u = 0; u < NU; ++u) gload1(ks, r, u);
  };
  // chunk j of a step into buffer buf: j < NWC a weight chunk (group j / 4 of the row, or
  // the thread's group), else token chunk j - NWC; each is 8 codes -> 16 bytes of fp16
  uint32_t tw[TN == 4 ? 2 : 1][2];                       // the groups' weight tables
  auto dq_chunk = [&](const W2Raw<TN>& r, int buf, int j) {
    uint8_t* const base = lds + buf * BUF;
    uint32_t o[4];
    if (j < NWC) {
      const int q = j >> 2, c = j & 3;
      if (c == 0) w2_group_table(lt, __ushort_as_half((unsigned short)r.s[q]), tw[q][0], tw[q][1]);
      dequant_w2((r.w[q][c >> 1] >> (16 * (c & 1))) & 0xFFFFu, tw[q][0], tw[q][1], o);
      const int slot = 4 * (TN == 4 ? q : wq) + c;
      *reinterpret_cast<v4u*>(base + A_OFF + wrow * RB + 16 * (slot ^ swa)) = v4u{o[0], o[1], o[2], o[3]};
    } else {
      const int q = (j - NWC) >> 2, c = (j - NWC) & 3;
      dequant_a4(r.x[q][c], lt, o);
      *reinterpret_cast<v4u*>(base + B_OFF + tid * RB + 16 * ((4 * q + c) ^ swb)) = v4u{o[0], o[1], o[2], o[3]};
    }
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wrow_a = wn * 32 * TN, wrow_b = wm * 128;
  // fragment i of a wave reads row wrow + 32 i + l32, whose swizzle (row & 7) is the lane's
  const int fa_off = A_OFF + (wrow_a + l32) * RB, fb_off = B_OFF + (wrow_b + l32) * RB, swl = l32 & 7;
  auto rd_a = [&](int buf, int sub, int i) {
    return *reinterpret_cast<const v8h*>(lds + buf * BUF + fa_off + 32 * RB * i + 16 * ((2 * sub + h) ^ swl));
  };
  auto rd_b = [&](int buf, int sub, int j) {
    return *reinterpret_cast<const v8h*>(lds + buf * BUF + fb_off + 32 * RB * j + 16 * ((2 * sub + h) ^ swl));
  };

  // step ks: products from buffer ks & 1, the codes of ks + 1 (in `cur`, loaded during step
  // ks - 1) dequantized into the other buffer, the loads of ks + 2 into `ld`.  The loop runs
  // two steps per iteration, so that the two register sets alternate without copies (a copy
  // would wait for the loads still in flight).  The buffer index is hidden from the compiler:
  // knowing it, it would keep both buffers' LDS addresses in registers and spill.
  auto step = [&](int ks, const W2Raw<TN>& cur, W2Raw<TN>& ld) {
    int buf = ks & 1;
    asm volatile("" : "+s"(buf));
    v8h fa[2][TN], fb[2][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i) fa[0][i] = rd_a(buf, 0, i);
#pragma unroll
    for (int j = 0; j < TM; ++j) fb[0][j] = rd_b(buf, 0, j);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int c = sub & 1, n = c ^ 1;
#pragma unroll
      for (int m = 0; m < TN * TM; ++m) {
        const int i = m / TM, j = m % TM;
        __builtin_amdgcn_sched_barrier(0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (sub < 3 && m < TN + TM) {
          if (m < TN) fa[n][m] = rd_a(buf, sub + 1, m);
          else fb[n][m - TN] = rd_b(buf, sub + 1, m - TN);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (w2_dq_at<TN>(TN * TM * sub + m) >= 0) {
          dq_chunk(cur, buf ^ 1, w2_dq_at<TN>(TN * TM * sub + m));
          __builtin_amdgcn_sched_barrier(0);
        }
        if (w2_load_at<TN>(sub, m) >= 0) {
          gload1(ks + 2, ld, w2_load_at<TN>(sub, m));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    lds_barrier();                                        // the next buffer is complete, this one free
  };

  W2Raw<TN> ra, rb;
  gload(0, ra);
  gload(1, rb);
#pragma unroll
  for (int j = 0; j < NWC + 8; ++j) dq_chunk(ra, 0, j);
  lds_barrier();
  // pairs of steps, then the last step when their number is odd (a conditional second step
  // inside the loop makes the register allocator copy the accumulators, and spill)
  int ks = 0;
  for (; ks + 1 < nks; ks += 2) {
    step(ks, rb, ra);
    step(ks + 1, ra, rb);
  }
  if (ks < nks) step(ks, rb, ra);

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

// The large-tile form's kernel: the first full_rows rows of 256 x 256 tiles take the full
// tile (walked column by column in groups of 8 along M, die-contiguous, as in the W4A4
// kernel), the tile rows below them, if any, tiles of half the width; with none of those,
// each workgroup loops over every grid-th tile.
__global__ __launch_bounds__(256, 1) void w2a4_gemm_big_kernel(
    const uint8_t* __restrict__ xcodes, const float* __restrict__ xscales, int M, int K,
    const uint8_t* __restrict__ wcodes, const __half* __restrict__ wscales, int N, LmTables lm,
    __half* __restrict__ Y, int full_rows) {
  __shared__ __align__(16) uint8_t lds[2 * 512 * 128];
  const LmRegTables lt = lm_reg_tables(lm);
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
    w2a4_big_tile<4>(lds, xcodes, xscales, M, K, wcodes, wscales, N, lt, Y, 256 * tile_m, 256 * tile_n);
  };
  if (full_rows == (M + 255) / 256) {
    // full tiles only: workgroup b takes tiles b, b + G, .. (G = the grid, a multiple of the 8
    // compute dies)
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
    w2a4_big_tile<2>(lds, xcodes, xscales, M, K, wcodes, wscales, N, lt, Y, 256 * tile_m, 128 * tile_n);
  }
}

hipError_t launch_w2a4_gemm(const uint8_t* xcodes, const float* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const __half* wscales, int64_t N, __half* Y, hipStream_t s) {
  // The large-tile form does a 256 x 256 tile in about the time of two rounds of 128 x 128
  // ones, and its rounds of tiles are four times coarser: it runs once the small tiles would
  // take more than two rounds (measured at K = 2240 and 5600: the small tiles win by 8-40%
  // up to 128 large tiles, the large ones by 12-70% from 144 up).  A last round that leaves
  // compute units idle goes to tiles of half the width when those fit in one round (as in
  // the W4A4 kernel); so does a grid of at most half a round when its half-width tiles fill
  // a quarter round or more (measured: they beat the small tiles by 2-25% from 64 of them
  // up, and lose by 2-7% at 18-36).
  const int64_t cus = device_cu_count();
  const int64_t tiles_n = (N + 255) / 256, tiles_m = (M + 255) / 256, tiles_n2 = (N + 127) / 128;
  const int64_t t256 = tiles_n * tiles_m;
  if (2 * t256 > cus || 4 * tiles_m * tiles_n2 >= cus) {
    const int64_t tail = t256 % cus;
    int64_t full_rows = tiles_m;
    if (tail > 0) {
      const int64_t hr = (tail + tiles_n - 1) / tiles_n;     // tile rows that hold the tail
      if (hr * tiles_n2 <= cus) full_rows = tiles_m - hr;
    }
    int64_t grid = tiles_n * full_rows + tiles_n2 * (tiles_m - full_rows);
    if (full_rows == tiles_m) {
      // no half-width tiles: even rounds, as in the W4A4 kernel
      const int64_t rounds = (t256 + cus - 1) / cus;
      const int64_t even = ((t256 + rounds - 1) / rounds + 7) / 8 * 8;
      if (even < grid) grid = even;
    }
    hipLaunchKernelGGL(w2a4_gemm_big_kernel, dim3((unsigned)grid), dim3(256), 0, s, xcodes, xscales, (int)M, (int)K,
                       wcodes, wscales, (int)N, lm_tables(), Y, (int)full_rows);
    return hipGetLastError();
  }
  constexpr int BN = 128, BM = 128, WN = 2, WM = 2;
  const int64_t tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  hipLaunchKernelGGL((w2a4_gemm_kernel<BN, BM, WN, WM>), dim3((unsigned)tiles), dim3(WN * WM * 64), 0, s, xcodes,
                     xscales, (int)M, (int)K, wcodes, wscales, (int)N, lm_tables(), Y);
  return hipGetLastError();
}

}  // namespace kq
