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
#include "kq_mfma_xform.hpp"

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

// Streaming Kronecker (or identity) + MXFP4 on the matrix cores: the activations are a
// flat sequence of 32-element blocks; a wavefront handles U chunks of 16 blocks (1 KiB)
// per step, each with one 16-byte load per lane, and writes 256 contiguous code bytes per
// chunk.  The next step's chunks are loaded while the current ones are transformed.
// KIND: 0 identity, 1 Kronecker A (x) B, 3 dense P (both through the hi + lo split).
// PTS (DMQ explainer, channel-wise power-of-two scaling): before the transform, input
// channel c is divided by 2^pts[c] in fp16 (exact unless the result is subnormal); channel
// c of block blk is (blk mod nbk) * 32 + its position in the block.
template <int U, int KIND, bool PTS>
__global__ __launch_bounds__(256) void kron_mx_mfma_stream_kernel(const uint4* __restrict__ X, int64_t nblocks,
                                                                  KronFactors f, const float* __restrict__ P,
                                                                  const int8_t* __restrict__ pts, int64_t nbk,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  constexpr bool KRON = KIND != 0;        // a general matrix: hi + lo products
  const int lane = threadIdx.x & 63, q = lane >> 4, bl = lane & 15;
  MfmaXform xf;
  if (KIND == 1) {
    xf = mfma_xform_kron(f, lane);
  } else if (KIND == 3) {
    xf = mfma_xform_dense(P, lane);
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
  // channel block of this lane's block: the blocks a lane visits advance by 16 nwaves,
  // so the block index modulo nbk is carried along instead of divided out each time.  The
  // exponents are fetched one step ahead (the table is small and stays in cache; the
  // fetch past the last step reads valid entries and is discarded).
  int32_t cb = 0, cstep = 0;
  uint2 ev[U];
  auto fetch_exponents = [&](uint2* e) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      e[u] = *reinterpret_cast<const uint2*>(pts + cb * 32 + 8 * q);     // exponents of the 8 channels
      cb += cstep;
      cb -= cb >= nbk ? (int32_t)nbk : 0;
    }
  };
  if (PTS) {
    cb = (int32_t)((wave * 16 + bl) % nbk);
    cstep = (int32_t)((nwaves * 16) % nbk);
    fetch_exponents(ev);
  }
  uint4 nxt[U];     // the chunks of the next step, in flight while this one is transformed
  auto load_step = [&](int64_t c0, uint4* r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * nwaves;
      const int64_t blk = c * 16 + bl;
      r[u] = (c < nchunks && blk < nblocks) ? X[blk * 4 + q] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (wave < nchunks) load_step(wave, nxt);
  for (int64_t c0 = wave; c0 < nchunks; c0 += nwaves * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = nxt[u];
    if (c0 + nwaves * U < nchunks) load_step(c0 + nwaves * U, nxt);
    uint2 ev_next[U];
    if (PTS) fetch_exponents(ev_next);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (PTS) raw[u] = pts_scale8(raw[u], ev[u]);
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
    if (PTS) {
#pragma unroll
      for (int u = 0; u < U; ++u) ev[u] = ev_next[u];
    }
  }
}

// Per-block Kronecker factors + MXFP4 on the matrix cores (KroQuant §02 with one (A, B)
// pair per block index instead of one per layer).  A matrix-core step transforms 16
// columns with one P, so a wavefront owns U consecutive block indices and a run of 8-row
// groups and takes them two block indices at a time: lane (q, c) holds quarter q of block
// (row 8 g + c % 8, index cb + c / 8), so one load instruction reads 8 rows x 128
// contiguous bytes (whole cache lines), the step runs once with P_cb and once with
// P_cb+1, and each lane keeps the result for its own index.  The fragments of the U
// indices are formed once per wavefront; the four wavefronts of a workgroup take
// consecutive runs, so per row a workgroup reads 4U consecutive blocks.
// AB: float [nbk][80] per block index: A (16, row-major) then B (64, row-major).
// PTS as in the streaming kernel; a lane's channels are fixed, so its exponents are read
// once.
template <int U, int G, bool PTS>
__global__ __launch_bounds__(256) void kron_blocks_mx_kernel(const uint4* __restrict__ X, int64_t M, int64_t nbk,
                                                             int64_t nseg, int64_t gps,
                                                             const float* __restrict__ AB,
                                                             const int8_t* __restrict__ pts,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  static_assert(U % 2 == 0, "block indices go in pairs");
  constexpr int NP = U / 2;
  const int lane = threadIdx.x & 63, q = lane >> 4, bl = lane & 15, rr = bl & 7, hf = bl >> 3;
  const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nrun = (nbk + U - 1) / U;                  // runs of U block indices
  if (wave >= nrun * nseg) return;                         // whole wavefronts only
  const int64_t cb0 = (wave % nrun) * U, seg = wave / nrun;
  MfmaXform xf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t cb = cb0 + u < nbk ? cb0 + u : nbk - 1;  // a run past the end repeats the last
    xf[u] = mfma_xform_kron_g(AB + cb * 80, lane);
  }
  uint2 ev[NP];                                            // this lane's exponents, per pair
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t cb = cb0 + 2 * p + hf < nbk ? cb0 + 2 * p + hf : nbk - 1;
    ev[p] = PTS ? *reinterpret_cast<const uint2*>(pts + cb * 32 + 8 * q) : make_uint2(0u, 0u);
  }
  const int64_t ngroups = (M + 7) >> 3;
  const int64_t g0 = seg * gps, g1 = g0 + gps < ngroups ? g0 + gps : ngroups;
  for (int64_t g = g0; g < g1; g += G) {               // G groups' loads in flight together
    uint4 raw[G][NP];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row = (g + h) * 8 + rr;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int64_t cb = cb0 + 2 * p + hf;
        raw[h][p] = (g + h < g1 && row < M && cb < nbk) ? X[(row * nbk + cb) * 4 + q] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row = (g + h) * 8 + rr;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (PTS) raw[h][p] = pts_scale8(raw[h][p], ev[p]);
        const v8h b = __builtin_bit_cast(v8h, raw[h][p]);
        float y0[8], y1[8], y[8];
        mfma_block_transform<true>(xf[2 * p], b, y0);
        mfma_block_transform<true>(xf[2 * p + 1], b, y1);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = (hf ? y1[i] : y0[i]) + 0.0f;   // an exact zero leaves as +0
        uint32_t w, sb;
        int off;
        mx_pack_block(y, q, w, off, sb);
        const int64_t cb = cb0 + 2 * p + hf;
        if (g + h < g1 && row < M && cb < nbk) {
          const int64_t blk = row * nbk + cb;
          *reinterpret_cast<uint32_t*>(codes + blk * 16 + off) = w;
          if (q == 0) scales[blk] = (uint8_t)sb;
        }
      }
    }
  }
}

// Row-group RPBH + MXFP4 on the matrix cores, optional centring.  R consecutive token
// rows are staged together in LDS, interleaved element by element ([k][r]: R halves per
// position), so one LDS read of 2R bytes gathers a permuted position for all R rows, and
// the gather table and sign masks (built once per persistent workgroup) serve R rows per
// read.  A workgroup of NW wavefronts holds one group: lane t loads 16-byte columns
// t, t + 64 NW of each of the R rows, transposes them in registers and writes them
// interleaved; the next group's columns are loaded while the current group is
// transformed.  Wavefront w transforms the 16-block chunks w and w + NW of all R rows.
// Centring is applied after the rotation: (x - mu 1) H32 = x H32 - 32 mu e_0 for the
// Sylvester matrix (every column but the first sums to zero), so only output 0 of each
// block is corrected; the result is the same linear map as centring first.
constexpr int RG_MAXW = 16;   // wavefronts per workgroup, at most
constexpr int RG_COLS = 2;    // 16-byte columns of a row per lane, at most (64 NW >= K / 16)
constexpr int RG_PV = 4;      // 16-byte perm chunks per lane in the set-up, at most

__host__ __device__ constexpr size_t rg_red_offset(int R, int K) {
  return ((size_t)R * K * 2 + (size_t)K * 2 + (size_t)(K / 32) * 4 + 15) & ~(size_t)15;
}
__host__ __device__ constexpr size_t rg_lds_bytes(int R, int K) { return rg_red_offset(R, K) + RG_MAXW * 16; }

template <int R>
struct GroupChunks {
  v4u v[RG_COLS][R];
};

// Columns col[] of rows row0 .. row0 + R - 1 (rows past M read row M - 1).
template <int R>
__device__ __forceinline__ GroupChunks<R> rg_load(const __half* X, int64_t row0, int64_t M, int K,
                                                  const int* col) {
  GroupChunks<R> g;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < M ? row0 + r : M - 1;
    const v4u* xr = reinterpret_cast<const v4u*>(X + row * (int64_t)K);
#pragma unroll
    for (int j = 0; j < RG_COLS; ++j) g.v[j][r] = xr[col[j]];
  }
  return g;
}

#define KQ_PERM_LO 0x05040100u   // (lo16 of s1, lo16 of s0)
#define KQ_PERM_HI 0x07060302u   // (hi16 of s1, hi16 of s0)

// Wavefronts per workgroup at most, by variant: the four-row Lloyd-Max form needs more
// registers and is only used up to K = 6144 (at most six wavefronts).
template <int R, int FMT>
constexpr int rg_maxw() { return (FMT == 1 && R == 4) ? 8 : RG_MAXW; }

template <int R, bool CENTER, int FMT>
__global__ __launch_bounds__((64 * rg_maxw<R, FMT>())) void rpbh_mx_group_kernel(
    const __half* X, int64_t M, int K, const int32_t* __restrict__ perm,
    const int8_t* __restrict__ sign, LmTables lm, uint8_t* __restrict__ codes, void* __restrict__ scales,
    __half* __restrict__ mu) {
  static_assert(R == 2 || R == 4, "rows per group");
  static_assert(FMT == 0 || !CENTER, "the Lloyd-Max output is offered without centring");
  constexpr bool RSUM = CENTER || FMT == 1;     // a per-row reduction over the staged row
  extern __shared__ __align__(16) unsigned char smem[];
  const int t = threadIdx.x, T = blockDim.x, NW = T >> 6, lane = t & 63, wid = t >> 6;
  const int q = lane >> 4, bl = lane & 15;
  const int cols = K >> 3, nb = K >> 5, nchunk = (nb + 15) >> 4;
  unsigned char* const slot = smem;                                                       // [K][R] halves
  uint16_t* const tab = reinterpret_cast<uint16_t*>(smem + (size_t)R * K * 2);            // [K]
  uint32_t* const smask = reinterpret_cast<uint32_t*>(smem + (size_t)R * K * 2 + (size_t)K * 2);   // [nb]
  float* const red = reinterpret_cast<float*>(smem + rg_red_offset(R, K));                // [NW][4]

  // this lane's columns (clamped: a lane past the end repeats the last column, whose
  // duplicate LDS writes carry identical data)
  int col[RG_COLS];
  bool colv[RG_COLS];
#pragma unroll
  for (int j = 0; j < RG_COLS; ++j) {
    const int c = t + T * j;
    colv[j] = c < cols;
    col[j] = colv[j] ? c : cols - 1;
  }
  const int64_t ngroups = (M + R - 1) / R;
  int64_t g = blockIdx.x;

  // set-up loads (perm chunks, the sign bytes of block t), then the first group's loads,
  // all in flight together; then the gather table and sign masks
  // (workgroups start the table at different chunks so that they do not all read the same
  // lines at the same moment)
  const int npc = K >> 2, rot = (int)((blockIdx.x * 61u) % (unsigned)npc);
  v4u pv[RG_PV];
  int pc[RG_PV];
#pragma unroll
  for (int i = 0; i < RG_PV; ++i) {
    const int c = min(t + T * i, npc - 1);
    pc[i] = c + rot < npc ? c + rot : c + rot - npc;
    pv[i] = reinterpret_cast<const v4u*>(perm)[pc[i]];
  }
  const int sbk = (int)((min(t, nb - 1) + blockIdx.x * 7u) % (unsigned)nb);
  uint32_t sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = reinterpret_cast<const uint32_t*>(sign + 32 * sbk)[i];
  GroupChunks<R> raw = rg_load<R>(X, g * R, M, K, col);
  // keep the group's loads ahead of the set-up's waits (X is not declared restrict, so
  // the compiler may not move its loads across this point)
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < RG_PV; ++i)
    reinterpret_cast<uint2*>(tab)[pc[i]] = make_uint2((pv[i].x & 0xFFFFu) | (pv[i].y << 16),
                                                      (pv[i].z & 0xFFFFu) | (pv[i].w << 16));
  {
    uint32_t m = 0;      // bit j: d_{32 b + j} < 0
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) m |= ((sv[i] >> (8 * k + 7)) & 1u) << (4 * i + k);
    smask[sbk] = m;
  }
  const MfmaXform xf = mfma_xform_hadamard(lane);

  for (; g < ngroups; g += gridDim.x) {
    lds_barrier();       // the previous group's gathers are done (and the table is written)
    float ps[R];
#pragma unroll
    for (int r = 0; r < R; ++r) ps[r] = 0.0f;
#pragma unroll
    for (int j = 0; j < RG_COLS; ++j) {
      const GroupChunks<R>& c = raw;
      v4u* dst = reinterpret_cast<v4u*>(slot) + (size_t)col[j] * (R * 8 * 2 / 16);
      if (R == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4u a = c.v[j][0], b = c.v[j][1], cc = c.v[j][R - 2], d = c.v[j][R - 1];
          dst[i] = v4u{__builtin_amdgcn_perm(b[i], a[i], KQ_PERM_LO), __builtin_amdgcn_perm(d[i], cc[i], KQ_PERM_LO),
                       __builtin_amdgcn_perm(b[i], a[i], KQ_PERM_HI), __builtin_amdgcn_perm(d[i], cc[i], KQ_PERM_HI)};
        }
      } else {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
          const v4u a = c.v[j][0], b = c.v[j][1];
          dst[m2] = v4u{__builtin_amdgcn_perm(b[2 * m2], a[2 * m2], KQ_PERM_LO),
                        __builtin_amdgcn_perm(b[2 * m2], a[2 * m2], KQ_PERM_HI),
                        __builtin_amdgcn_perm(b[2 * m2 + 1], a[2 * m2 + 1], KQ_PERM_LO),
                        __builtin_amdgcn_perm(b[2 * m2 + 1], a[2 * m2 + 1], KQ_PERM_HI)};
        }
      }
      if (RSUM) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float s8 = 0.0f;     // sum of the 8 halves (centring) or of their squares (Lloyd-Max scale)
#pragma unroll
          for (int m = 0; m < 4; ++m) s8 = FMT == 1 ? sq_f16x2(c.v[j][r][m], s8) : add_f16x2(c.v[j][r][m], s8);
          ps[r] += colv[j] ? s8 : 0.0f;     // a repeated column is not counted
        }
      }
    }
    if (g + gridDim.x < ngroups) raw = rg_load<R>(X, (g + gridDim.x) * R, M, K, col);   // prefetch the next group
    if (RSUM) {
      // wave sums of the R partial sums in registers: each lane-half / lane-row swap adds
      // the partner's copy of one value while halving the set (the swap returns, per lane,
      // its own value in one result and the partner's in the other), then a row sum;
      // lanes of 16-lane row j end with the sum of row j (R = 4) or j / 2 (R = 2)
      float v;
      if (R == 4) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps[0]), __float_as_uint(ps[2]), false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps[1]), __float_as_uint(ps[R - 1]), false, false);
        const float k0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);   // rows 0 (lanes < 32) / 2
        const float k1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);   // rows 1 / 3
        const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
        v = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      } else {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps[0]), __float_as_uint(ps[1]), false, false);
        const float k = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(k), __float_as_uint(k), false, false);
        v = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      }
      v = row16_sum(v);
      if ((lane & 15) == 0 && (R == 4 || (lane & 16) == 0)) red[wid * 4 + (R == 4 ? (lane >> 4) : (lane >> 5))] = v;
    }
    lds_barrier();       // the group is staged (and the partial sums are visible)
    float m32[R], scr[R];          // the centring term, or the Lloyd-Max scale, per row
#pragma unroll
    for (int r = 0; r < R; ++r) m32[r] = scr[r] = 0.0f;
    if (RSUM) {
      float tot[R];
#pragma unroll
      for (int r = 0; r < R; ++r) tot[r] = 0.0f;
      for (int w = 0; w < NW; ++w) {
        const float4 rw = reinterpret_cast<const float4*>(red)[w];
        tot[0] += rw.x;
        tot[1] += rw.y;
        if (R == 4) {
          tot[2 % R] += rw.z;
          tot[3 % R] += rw.w;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (FMT == 1) {
          // s_t = RMS of the rotated token = ||x_t|| / sqrt(K), the rotation being
          // orthogonal
          scr[r] = sqrtf(tot[r] / (float)K);
          if (t == r && g * R + r < M) reinterpret_cast<float*>(scales)[g * R + r] = scr[r];
        } else {
          const __half mh = __float2half_rn(tot[r] / (float)K);
          m32[r] = 32.0f * __half2float(mh);
          if (t == r && g * R + r < M) mu[g * R + r] = mh;
        }
      }
    }
    // the group's rows of codes and scales (rows past M are outside both ranges)
    const int64_t nrows = M - g * R < R ? M - g * R : R;
    const __amdgpu_buffer_rsrc_t rcodes = make_rsrc(codes + g * R * (int64_t)(K >> 1), nrows * (K >> 1));
    const __amdgpu_buffer_rsrc_t rscales =
        make_rsrc(static_cast<uint8_t*>(scales) + (FMT == 0 ? g * R * (int64_t)nb : 0), FMT == 0 ? nrows * nb : 0);
#pragma unroll 1
    for (int it = 0; it < 2; ++it) {
      const int ch = wid + NW * it;
      if (ch >= nchunk) break;
      const int blk = 16 * ch + bl;
      const bool bv = blk < nb;
      const int bb = bv ? blk : nb - 1;          // lanes past the row's end gather a real block, not stored
      const v4u ix = *reinterpret_cast<const v4u*>(tab + 32 * bb + 8 * q);
      uint32_t pos[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pos[2 * i] = ix[i] & 0xFFFFu;
        pos[2 * i + 1] = ix[i] >> 16;
      }
      v4u bop[R];      // B operands (8 fp16 inputs of block bb) of the R rows
      if (R == 4) {
        uint2 gv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = *reinterpret_cast<const uint2*>(slot + (size_t)pos[i] * 8);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          bop[0][m] = __builtin_amdgcn_perm(gv[2 * m + 1].x, gv[2 * m].x, KQ_PERM_LO);
          bop[1][m] = __builtin_amdgcn_perm(gv[2 * m + 1].x, gv[2 * m].x, KQ_PERM_HI);
          bop[2][m] = __builtin_amdgcn_perm(gv[2 * m + 1].y, gv[2 * m].y, KQ_PERM_LO);
          bop[R - 1][m] = __builtin_amdgcn_perm(gv[2 * m + 1].y, gv[2 * m].y, KQ_PERM_HI);
        }
      } else {
        uint32_t gv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = *reinterpret_cast<const uint32_t*>(slot + (size_t)pos[i] * 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          bop[0][m] = __builtin_amdgcn_perm(gv[2 * m + 1], gv[2 * m], KQ_PERM_LO);
          bop[1][m] = __builtin_amdgcn_perm(gv[2 * m + 1], gv[2 * m], KQ_PERM_HI);
        }
      }
      const uint32_t sm = smask[bb];
      float coef[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = (i < 4 ? 4 * q + i : 16 + 4 * q + (i - 4));
        coef[i] = ((sm >> j) & 1u) ? -KQ_INV_SQRT32 : KQ_INV_SQRT32;
      }
      // all R transforms first, then the packing, then branch-free stores (masked lanes
      // and rows past M fall outside the buffer ranges), so the R rows' chains interleave
      float y[R][8];
#pragma unroll
      for (int r = 0; r < R; ++r) mfma_block_transform<false>(xf, __builtin_bit_cast(v8h, bop[r]), y[r]);
      uint32_t w[R], sb[R];
      int off = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (CENTER && q == 0) y[r][0] -= m32[r];      // output 0 of the block
#pragma unroll
        for (int i = 0; i < 8; ++i) y[r][i] = __builtin_fmaf(y[r][i], coef[i], 0.0f);   // +0 for an exact zero
        if (FMT == 1) {
          float ts[7];                                  // the thresholds scaled by the row's s_t
#pragma unroll
          for (int i = 0; i < 7; ++i) ts[i] = lm.t16[i] * scr[r];
          lm_pack_block(y[r], q, ts, w[r], off);
        }
        else mx_pack_block(y[r], q, w[r], off, sb[r]);
      }
      const int coff = bv ? 16 * blk + off : KQ_OOB;
      const int soff = (bv && q == 0) ? blk : KQ_OOB;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        __builtin_amdgcn_raw_buffer_store_b32(w[r], rcodes, coff + (coff == KQ_OOB ? 0 : r * (K >> 1)), 0, 0);
        if (FMT == 0)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb[r], rscales, soff + (soff == KQ_OOB ? 0 : r * nb), 0, 0);
      }
    }
  }
}

// Persistent workgroups: one per U chunks of each wavefront, at most as many as are
// resident at once (a grid past that would run its last workgroups in a partial second
// round, each with a full share of the chunks).
template <int U, int KIND, bool PTS>
static void stream_launch(int64_t nblocks, hipStream_t s, const uint4* X, const KronFactors& f, const float* P,
                          const int8_t* pts, int64_t nbk, uint8_t* codes, uint8_t* scales) {
  const auto kern = kron_mx_mfma_stream_kernel<U, KIND, PTS>;
  const int64_t nchunks = (nblocks + 15) / 16;
  const int64_t waves = (nchunks + U - 1) / U;
  int64_t grid = (waves + 3) / 4;
  const int64_t cap =
      (int64_t)device_cu_count() * resident_blocks_per_cu(reinterpret_cast<const void*>(kern), 256, 0);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, X, nblocks, f, P, pts, nbk, codes, scales);
}

template <int U, int KIND>
static void stream_launch(int64_t nblocks, hipStream_t s, const uint4* X, const KronFactors& f, const float* P,
                          const int8_t* pts, int64_t nbk, uint8_t* codes, uint8_t* scales) {
  if (pts) stream_launch<U, KIND, true>(nblocks, s, X, f, P, pts, nbk, codes, scales);
  else stream_launch<U, KIND, false>(nblocks, s, X, f, P, pts, nbk, codes, scales);
}

// Two chunks per step with the next step's loads in flight (as many registers as four
// chunks without them, so as many workgroups stay resident): against four chunks without,
// 4-11% faster from M = 4608, K = 3072 to M = 8192, K = 4608 and equal at M = 8192,
// K = 1152 and M = 17550, K = 3072; with one chunk per step (eight resident workgroups per
// compute unit instead of five) the large shapes were 2-10% slower on one of three GPUs.
hipError_t launch_kron_mx_mfma(int kind, const __half* X, int64_t nblocks, const KronFactors& f, const float* P,
                               const int8_t* pts, int64_t nbk, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  constexpr int U = 2;
  const uint4* Xv = reinterpret_cast<const uint4*>(X);
  if (kind == 1) stream_launch<U, 1>(nblocks, s, Xv, f, P, pts, nbk, codes, scales);
  else if (kind == 3) stream_launch<U, 3>(nblocks, s, Xv, f, P, pts, nbk, codes, scales);
  else stream_launch<U, 0>(nblocks, s, Xv, f, P, pts, nbk, codes, scales);
  return hipGetLastError();
}

// Per-block factors: ceil(nbk / U) * nseg wavefronts, segment s of a run taking the 8-row
// groups [s gps, (s + 1) gps); at most as many wavefronts as are resident at once, so that
// no partial second round of workgroups follows the first.
template <bool PTS>
static void kron_blocks_launch(const uint4* X, int64_t M, int64_t K, const float* AB, const int8_t* pts,
                               uint8_t* codes, uint8_t* scales, hipStream_t s) {
  constexpr int U = 4, G = 2;
  const auto kern = kron_blocks_mx_kernel<U, G, PTS>;
  const int64_t nbk = K / 32, nrun = (nbk + U - 1) / U, ngroups = (M + 7) / 8;
  const int64_t target =
      (int64_t)device_cu_count() * resident_blocks_per_cu(reinterpret_cast<const void*>(kern), 256, 0) * 4;
  int64_t nseg = target / nrun;
  if (nseg > ngroups) nseg = ngroups;
  if (nseg < 1) nseg = 1;
  const int64_t gps = (ngroups + nseg - 1) / nseg;
  nseg = (ngroups + gps - 1) / gps;                        // no empty segment
  hipLaunchKernelGGL(kern, dim3((unsigned)((nrun * nseg + 3) / 4)), dim3(256), 0, s, X, M, nbk, nseg, gps, AB, pts,
                     codes, scales);
}

hipError_t launch_kron_blocks_mx(const __half* X, int64_t M, int64_t K, const float* AB, const int8_t* pts,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const uint4* Xv = reinterpret_cast<const uint4*>(X);
  if (pts) kron_blocks_launch<true>(Xv, M, K, AB, pts, codes, scales, s);
  else kron_blocks_launch<false>(Xv, M, K, AB, pts, codes, scales, s);
  return hipGetLastError();
}


template <int R, bool CENTER, int FMT>
static hipError_t rpbh_group_launch(const __half* X, int64_t M, int K, const int32_t* perm, const int8_t* sign,
                                    uint8_t* codes, void* scales, __half* mu, hipStream_t s) {
  // wavefronts: enough that each transforms at most two 16-block chunks of the group
  // (this also keeps the set-up at <= 4 perm chunks and the staging at <= 2 columns per
  // lane); persistent workgroups, as many as are resident at once
  const int nchunk = (K / 32 + 15) / 16;
  const int nw = (nchunk + 1) / 2;
  if (nw > rg_maxw<R, FMT>()) return hipErrorInvalidValue;
  const unsigned threads = 64u * (unsigned)nw;
  const size_t lds = rg_lds_bytes(R, K);
  const auto kern = rpbh_mx_group_kernel<R, CENTER, FMT>;
  int64_t grid = (M + R - 1) / R;
  const int64_t cap =
      (int64_t)device_cu_count() * resident_blocks_per_cu(reinterpret_cast<const void*>(kern), (int)threads, lds);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, s, X, M, K, perm, sign, lm_tables(), codes, scales,
                     mu);
  return hipGetLastError();
}

hipError_t launch_rpbh_mx_mfma(bool center, const __half* X, int64_t M, int64_t K, const int32_t* perm,
                               const int8_t* sign, uint8_t* codes, uint8_t* scales, __half* mu, hipStream_t s) {
  if (K > 16384) return hipErrorInvalidValue;
  // four rows per group up to K = 6144; above, two, which halves the staging so that two
  // workgroups share a compute unit (at K = 12288 that measured 13% faster than four rows
  // with one workgroup per compute unit)
  if (K <= 6144)
    return center ? rpbh_group_launch<4, true, 0>(X, M, (int)K, perm, sign, codes, scales, mu, s)
                  : rpbh_group_launch<4, false, 0>(X, M, (int)K, perm, sign, codes, scales, mu, s);
  return center ? rpbh_group_launch<2, true, 0>(X, M, (int)K, perm, sign, codes, scales, mu, s)
                : rpbh_group_launch<2, false, 0>(X, M, (int)K, perm, sign, codes, scales, mu, s);
}

// Lloyd-Max form: four rows per group up to K = 2048, two above (with their larger
// register set four rows measured 4% slower than two at K = 2240 and 37% at K = 5600).
hipError_t launch_rpbh_lm4_mfma(const __half* X, int64_t M, int64_t K, const int32_t* perm, const int8_t* sign,
                                uint8_t* codes, float* scales, hipStream_t s) {
  if (K > 16384) return hipErrorInvalidValue;
  if (K <= 2048) return rpbh_group_launch<4, false, 1>(X, M, (int)K, perm, sign, codes, scales, nullptr, s);
  return rpbh_group_launch<2, false, 1>(X, M, (int)K, perm, sign, codes, scales, nullptr, s);
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
