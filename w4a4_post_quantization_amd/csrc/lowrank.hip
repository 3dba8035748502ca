// Low-rank down-projection of the SVDQuant branch (explainer §3): T = X L1^T, fp16
// matrix cores with fp32 accumulation, T stored as fp16 [M][r] (the branch is held in
// 16 bits).  X is the original fp16 activation [M][K], L1 is [r][K].
//
// A workgroup of SPLIT wavefronts owns 16 rows; wavefront w reduces the 32-wide k-steps
// w, w+SPLIT, ... with v_mfma_f32_16x16x32_f16 (lane l: row l%16, k = 8*(l/16)..+7, one
// 16-byte load per operand).  Loads are issued in batches of BATCH k-steps ahead of their
// MFMAs so each wavefront keeps several KiB in flight; the SPLIT partial 16 x r tiles are
// summed through LDS in a fixed order.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

template <int RT, int SPLIT, int BATCH>  // RT = r / 16 output tiles
__global__ __launch_bounds__(64 * SPLIT, 1) void lowrank_down_kernel(const __half* __restrict__ X,
                                                                  const __half* __restrict__ L1, int64_t M,
                                                                  int64_t K, __half* __restrict__ T) {
  __shared__ float part[SPLIT][16][RT * 16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  int64_t row = m0 + (lane & 15);
  if (row >= M) row = M - 1;  // clamp: the tail rows compute duplicates that are not stored
  const int q = lane >> 4;
  const int64_t nk = K >> 5;
  v4f acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  const __half* xr = X + row * K + 8 * q;
  const __half* lr[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) lr[t] = L1 + (int64_t)(16 * t + (lane & 15)) * K + 8 * q;
  // workgroups start at different k-steps so that they do not all read the same lines of
  // L1 at the same moment (a rotation of the k order; the sum is over the same terms)
  const int64_t rot = ((int64_t)blockIdx.x * 7 * SPLIT) % nk;
  for (int64_t s0 = w; s0 < nk; s0 += SPLIT * BATCH) {
    v8h a[BATCH], b[BATCH][RT];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t s = s0 + (int64_t)u * SPLIT;
      const bool ok = s < nk;
      int64_t ks = s + rot;
      ks = ks >= nk ? ks - nk : ks;
      a[u] = ok ? *reinterpret_cast<const v8h*>(xr + 32 * ks) : v8h{};
#pragma unroll
      for (int t = 0; t < RT; ++t) b[u][t] = ok ? *reinterpret_cast<const v8h*>(lr[t] + 32 * ks) : v8h{};
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[u], b[u][t], acc[t], 0, 0, 0);
  }
  // acc[t][i] = partial T[m0 + 4q + i][16t + lane%16]
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[w][4 * q + i][16 * t + (lane & 15)] = acc[t][i];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * RT * 16; e += 64 * SPLIT) {
    const int r = e / (RT * 16), c = e % (RT * 16);
    float v = 0.0f;
#pragma unroll
    for (int p = 0; p < SPLIT; ++p) v += part[p][r][c];
    if (m0 + r < M) T[(m0 + r) * (RT * 16) + c] = __float2half_rn(v);
  }
}

template <int SPLIT>
static hipError_t lowrank_launch(const __half* X, const __half* L1, int64_t M, int64_t K, int r, __half* T,
                                 hipStream_t s) {
  const dim3 grid((unsigned)((M + 15) / 16)), block(64 * SPLIT);
  switch (r) {
    case 16: hipLaunchKernelGGL((lowrank_down_kernel<1, SPLIT, 8>), grid, block, 0, s, X, L1, M, K, T); break;
    case 32: hipLaunchKernelGGL((lowrank_down_kernel<2, SPLIT, 8>), grid, block, 0, s, X, L1, M, K, T); break;
    case 64: hipLaunchKernelGGL((lowrank_down_kernel<4, SPLIT, 4>), grid, block, 0, s, X, L1, M, K, T); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lowrank_down(const __half* X, const __half* L1, int64_t M, int64_t K, int r, __half* T,
                               hipStream_t s) {
  // one batch of 8 k-steps per wavefront for K up to 8 x 32 x SPLIT; long rows use 16
  // wavefronts so each still issues its loads in one or two batches
  if (K >= 8192) return lowrank_launch<16>(X, L1, M, K, r, T, s);
  return lowrank_launch<8>(X, L1, M, K, r, T, s);
}

}  // namespace kq
