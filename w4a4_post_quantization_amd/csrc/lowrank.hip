// Low-rank down-projection of the SVDQuant branch (explainer §3): T = X L1^T, fp16
// matrix cores with fp32 accumulation, T stored as fp16 [M][r] (the branch is held in
// 16 bits).  X is the original fp16 activation [M][K], L1 is [r][K].
//
// The projection only streams X (r is small), so the kernel is built for HBM bandwidth:
//   - a workgroup owns 64 rows and a slice of K (split-K), so L1 is re-read once per 64
//     rows and the grid fills the compute units;
//   - X and L1 go from global memory straight into LDS in 128-wide k-chunks (buffer loads
//     with the LDS destination, full 128-byte lines), NS chunks deep;
//   - each of the four wavefronts owns 16 rows and all r columns: v_mfma_f32_16x16x32_f16
//     (lane l: row l%16, eight consecutive k of the 16-byte piece 4 s + l/16 of the chunk);
//   - with several K slices the fp32 partial tiles go to the caller's workspace and a
//     second, small kernel sums them in slice order (deterministic) and stores T.  (Summing them in the
//     last workgroup to finish a row block would need device-scope fences, which on this
//     chip write back and invalidate the whole L2 of the compute die: far slower.)
//
// The same kernel can also quantize what it streams (XK >= 0): the A fragment of each
// 32-wide step is, lane for lane, the B operand of the matrix-core block transform (16
// rows of one block index as the 16 blocks), so the chunk in LDS is transformed and
// packed to MXFP4 as well, and X is read once for both (SVDQuant explainer §3: the
// down-projection shares its input with the 4-bit branch).  XK: -1 none, 0 identity,
// 1 Kronecker A (x) B, 3 dense P; MXFP4 without centring.
#include "kq_device.hpp"
#include "kq_launch.hpp"
#include "kq_mfma_xform.hpp"

#include <algorithm>

namespace kq {

constexpr int LR_ROWS = 64;      // rows per workgroup
constexpr int LR_KC = 128;       // k per chunk (256 bytes of a row)

// 16-byte piece c of a 256-byte LDS row sits at slot c ^ (row % 16): the fragment reads
// (16 rows x one piece) then touch 16 distinct bank groups.
__device__ __forceinline__ int lr_slot(int row, int piece) { return piece ^ (row & 15); }

template <int RR, int NS>
struct LrCfg {
  static constexpr int RT = RR / 16;                    // 16-column output tiles
  static constexpr int X_BYTES = LR_ROWS * 256;         // one chunk of X
  static constexpr int STAGE = X_BYTES + RR * 256;      // ... and of L1
  static constexpr int LDS = NS * STAGE;
  static constexpr int LPW = 4 + RR / 16;               // load instructions per wave per chunk
  static constexpr int SPW = 8;                         // store instructions per wave per chunk (fused form)
};

template <int RR, int NS, int XK>
__global__ __launch_bounds__(256) void lowrank_down_kernel(const __half* __restrict__ X,
                                                           const __half* __restrict__ L1, int M, int K,
                                                           int slices, int cps, float* __restrict__ part,
                                                           __half* __restrict__ T, KronFactors fk,
                                                           const float* __restrict__ P,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  using C = LrCfg<RR, NS>;
  __shared__ __align__(16) uint8_t lds[C::LDS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rb = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int m0 = rb * LR_ROWS;
  const int nch = (K + LR_KC - 1) / LR_KC;
  const int c0 = sl * cps;                                   // first chunk of the slice
  const int nc = max(0, min(cps, nch - c0));                 // chunks in the slice

  const v4i rX = rsrc_words(X + (int64_t)m0 * K, (int64_t)(M - m0) * K * 2);   // rows past M read zeros
  const v4i rL = rsrc_words(L1, (int64_t)RR * K * 2);
  const uint32_t lds0 = lds_addr(lds);

  // load instruction j of this wave covers 4 rows x 256 bytes: row 4 j' + lane / 16 of
  // its operand (j' numbering the instruction within the operand), LDS slot lane % 16,
  // which holds the global piece slot ^ (row % 16)
  int xoff[4], loff[RR / 16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * w + 4 * j + (lane >> 4);
    const int piece = (lane & 15) ^ (row & 15);
    xoff[j] = (row * K + 8 * piece) * 2;
  }
#pragma unroll
  for (int j = 0; j < RR / 16; ++j) {
    const int row = (RR / 4) * w + 4 * j + (lane >> 4);      // RR / 4 rows of L1 per wave
    const int piece = (lane & 15) ^ (row & 15);
    loff[j] = (row * K + 8 * piece) * 2;
  }
  auto issue = [&](int f) {                                  // chunk f of the slice into stage f % NS
    const uint32_t st = lds0 + (uint32_t)((f % NS) * C::STAGE);
    const int kbase = (c0 + f) * LR_KC;
    const bool live = f < nc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * w + 4 * j + (lane >> 4);
      const int k = kbase + 8 * ((lane & 15) ^ (row & 15));
      lds_load16(rX, st + (16 * w + 4 * j) * 256, live && k < K ? xoff[j] + kbase * 2 : KQ_OOB);
    }
#pragma unroll
    for (int j = 0; j < RR / 16; ++j) {
      const int row = (RR / 4) * w + 4 * j + (lane >> 4);
      const int k = kbase + 8 * ((lane & 15) ^ (row & 15));
      lds_load16(rL, st + C::X_BYTES + ((RR / 4) * w + 4 * j) * 256, live && k < K ? loff[j] + kbase * 2 : KQ_OOB);
    }
  };

  v4f acc[C::RT];
#pragma unroll
  for (int t = 0; t < C::RT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  MfmaXform xf;
  if (XK == 1) xf = mfma_xform_kron(fk, lane);
  else if (XK == 3) xf = mfma_xform_dense(P, lane);
  else if (XK == 0) {   // identity: P^T rows are unit vectors
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xf.a[t][0][i] = (16 * t + (lane & 15) == 8 * (lane >> 4) + i) ? (_Float16)1.0f : (_Float16)0.0f;
        xf.a[t][1][i] = (_Float16)0.0f;
      }
  }
  const int nbk = K >> 5;
  // the fused form's codes and scales of this row block (rows past M are outside both ranges)
  const __amdgpu_buffer_rsrc_t rcodes = make_rsrc(codes + (int64_t)m0 * (K >> 1), (int64_t)(M - m0) * (K >> 1));
  const __amdgpu_buffer_rsrc_t rscales = make_rsrc(scales + (int64_t)m0 * nbk, (int64_t)(M - m0) * nbk);

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p);
  const int arow = 16 * w + (lane & 15);
  for (int f = 0; f < nc; ++f) {
    // chunk f has landed once at most the operations issued after its loads are outstanding:
    // the NS - 2 younger chunks' loads and, in the fused form, the SPW stores (all issued,
    // masked lanes out of range) of each chunk processed since (at most NS - 1)
    if (XK < 0 || f == 0) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * C::LPW));
    } else if (NS == 2 || f == 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * C::LPW + C::SPW));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * C::LPW + 2 * C::SPW));
    }
    lds_barrier();                                           // ... for every wave; stage (f - 1) % NS is free
    issue(f + NS - 1);
    const uint8_t* st = lds + (f % NS) * C::STAGE;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int piece = 4 * s + (lane >> 4);
      const v8h a = *reinterpret_cast<const v8h*>(st + arow * 256 + 16 * lr_slot(arow, piece));
#pragma unroll
      for (int t = 0; t < C::RT; ++t) {
        const int n = 16 * t + (lane & 15);
        const v8h b = *reinterpret_cast<const v8h*>(st + C::X_BYTES + n * 256 + 16 * lr_slot(n, piece));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
      }
      if (XK >= 0) {                 // block (c0 + f) * 4 + s of rows m0 + 16 w + lane % 16
        float y[8];
        mfma_block_transform<(XK > 0)>(xf, a, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] += 0.0f;    // an exact zero leaves as +0
        uint32_t wd, sb;
        int off;
        mx_pack_block(y, lane >> 4, wd, off, sb);
        // one code and one scale store per step, whatever the lanes hold (the wait above
        // counts them)
        const int kb = (c0 + f) * 4 + s;
        const int blk = arow * nbk + kb;                     // within the row block
        __builtin_amdgcn_raw_buffer_store_b32(wd, rcodes, kb < nbk ? blk * 16 + off : KQ_OOB, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rscales, kb < nbk && (lane >> 4) == 0 ? blk : KQ_OOB, 0,
                                             0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                 // no load may land after the workgroup ends

  // acc[t][i] = (partial) T[m0 + 16 w + 4 (lane / 16) + i][16 t + lane % 16]
  const int orow = 16 * w + 4 * (lane >> 4);
  if (slices == 1) {
#pragma unroll
    for (int t = 0; t < C::RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m0 + orow + i < M) T[(int64_t)(m0 + orow + i) * RR + 16 * t + (lane & 15)] = __float2half_rn(acc[t][i]);
    return;
  }
  float* const mine = part + ((int64_t)sl * M + m0) * RR;
#pragma unroll
  for (int t = 0; t < C::RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + orow + i < M) mine[(orow + i) * RR + 16 * t + (lane & 15)] = acc[t][i];
}

// T[m][c] = fp16(sum over slices s, in order, of part[s][m][c]); four columns per thread.
// The slices' loads go out eight at a time (range-checked: those past the last slice read
// zeros, which leave the sum unchanged), so a thread waits one memory latency per eight
// slices instead of one per slice.
constexpr int LR_RED_THREADS = 64;
constexpr int LR_RED_BATCH = 8;

template <int RR>
__global__ __launch_bounds__(LR_RED_THREADS) void lowrank_reduce_kernel(const float* __restrict__ part, int M,
                                                                        int slices, __half* __restrict__ T) {
  const int e = (blockIdx.x * LR_RED_THREADS + threadIdx.x) * 4;   // first of four elements
  if (e >= M * RR) return;
  const int plane = M * RR * 4;                                     // bytes per slice
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, (int64_t)slices * plane);
  v4f v = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < slices; s0 += LR_RED_BATCH) {
    v4f t[LR_RED_BATCH];
#pragma unroll
    for (int j = 0; j < LR_RED_BATCH; ++j)
      t[j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rp, (s0 + j) * plane + 4 * e, 0, 0));
    v = s0 == 0 ? t[0] : v + t[0];
#pragma unroll
    for (int j = 1; j < LR_RED_BATCH; ++j) v += t[j];
  }
  const __half2 h0 = __floats2half2_rn(v[0], v[1]), h1 = __floats2half2_rn(v[2], v[3]);
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  *reinterpret_cast<v2u*>(T + e) = v2u{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
}

// Slices of K per 64-row block: with fewer row blocks than compute units, as many as fill
// the compute units once (at M = 4608, 3 slices, 216 workgroups, against 6 and 15 before:
// the FLUX-like step 3.8 us faster); with more, enough workgroups for every compute unit to
// hold a few.  A slice has at least four chunks, and (with `cap` bytes of workspace) the
// partials fit.
static int lr_slices(int64_t M, int64_t K, int r, size_t cap) {
  const int64_t blocks = (M + LR_ROWS - 1) / LR_ROWS;
  const int64_t nch = (K + LR_KC - 1) / LR_KC;
  const int64_t cus = device_cu_count();
  int64_t s = blocks < cus ? cus / blocks : (4 * cus + blocks - 1) / blocks;
  s = std::min<int64_t>(s, std::max<int64_t>(1, nch / 4));
  while (s > 1 && (size_t)(s * M * r * 4) > cap) --s;
  return (int)std::max<int64_t>(s, 1);
}

size_t lowrank_workspace_bytes(int64_t M, int64_t K, int r) {
  const int s = lr_slices(M, K, r, ~(size_t)0);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)r * 4 : 0;
}

// Workspace of the linear that runs the down-projection itself: T (fp16 [M][r], padded to
// 256 bytes) followed by the partial sums of as many slices as any K could use (the slice
// count is capped by the compute-unit count against the row blocks, not by K).
size_t lowrank_t_bytes(int64_t M, int r) { return ((size_t)M * (size_t)r * 2 + 255) & ~(size_t)255; }
size_t lowrank_linear_workspace_bytes(int64_t M, int r) {
  if (r == 0) return 0;
  const int s = lr_slices(M, INT64_MAX / 4, r, ~(size_t)0);
  return lowrank_t_bytes(M, r) + (s > 1 ? (size_t)s * (size_t)M * (size_t)r * 4 : 0);
}

template <int RR, int XK>
static hipError_t lowrank_launch(const __half* X, const __half* L1, int64_t M, int64_t K, __half* T, float* part,
                                 hipStream_t s, int slices, const KronFactors& fk, const float* P, uint8_t* codes,
                                 uint8_t* scales) {
  constexpr int NS = RR == 64 ? 2 : 3;
  const int64_t blocks = (M + LR_ROWS - 1) / LR_ROWS;
  const int64_t nch = (K + LR_KC - 1) / LR_KC;
  const int cps = (int)((nch + slices - 1) / slices);
  slices = (int)((nch + cps - 1) / cps);                     // no empty slice (never more)
  hipLaunchKernelGGL((lowrank_down_kernel<RR, NS, XK>), dim3((unsigned)(blocks * slices)), dim3(256), 0, s, X, L1,
                     (int)M, (int)K, slices, cps, part, T, fk, P, codes, scales);
  if (slices > 1) {
    // the reduction addresses the partial sums with 32-bit offsets (the split only runs
    // while the row blocks are fewer than four per compute unit, so they are small)
    if ((int64_t)(slices + LR_RED_BATCH) * M * RR * 4 > INT32_MAX) return hipErrorInvalidValue;
    const int64_t threads = M * RR / 4;
    hipLaunchKernelGGL((lowrank_reduce_kernel<RR>), dim3((unsigned)((threads + LR_RED_THREADS - 1) / LR_RED_THREADS)),
                       dim3(LR_RED_THREADS), 0, s, part, (int)M, slices, T);
  }
  return hipGetLastError();
}

template <int XK>
static hipError_t lowrank_rank(const __half* X, const __half* L1, int64_t M, int64_t K, int r, __half* T, float* part,
                               hipStream_t s, int slices, const KronFactors& fk, const float* P, uint8_t* codes,
                               uint8_t* scales) {
  switch (r) {
    case 16: return lowrank_launch<16, XK>(X, L1, M, K, T, part, s, slices, fk, P, codes, scales);
    case 32: return lowrank_launch<32, XK>(X, L1, M, K, T, part, s, slices, fk, P, codes, scales);
    case 48: return lowrank_launch<48, XK>(X, L1, M, K, T, part, s, slices, fk, P, codes, scales);
    case 64: return lowrank_launch<64, XK>(X, L1, M, K, T, part, s, slices, fk, P, codes, scales);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lowrank_down(const __half* X, const __half* L1, int64_t M, int64_t K, int r, __half* T,
                               float* part, size_t part_bytes, hipStream_t s) {
  const int slices = part ? lr_slices(M, K, r, part_bytes) : 1;
  const KronFactors none{};
  return lowrank_rank<-1>(X, L1, M, K, r, T, part, s, slices, none, nullptr, nullptr, nullptr);
}

hipError_t launch_lowrank_xform_mx(int kind, const __half* X, const __half* L1, int64_t M, int64_t K, int r,
                                   __half* T, float* part, size_t part_bytes, const KronFactors& fk, const float* P,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int slices = part ? lr_slices(M, K, r, part_bytes) : 1;
  if (kind == 1) return lowrank_rank<1>(X, L1, M, K, r, T, part, s, slices, fk, P, codes, scales);
  if (kind == 3) return lowrank_rank<3>(X, L1, M, K, r, T, part, s, slices, fk, P, codes, scales);
  return lowrank_rank<0>(X, L1, M, K, r, T, part, s, slices, fk, P, codes, scales);
}

}  // namespace kq
