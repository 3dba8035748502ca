// Measurement helpers outside the activation path.
//   - The shader clock as the chip runs it: one wavefront counts shader-clock cycles
//     (s_memtime) against the constant 100 MHz reference counter (s_memrealtime) for a
//     requested span of reference time; launched on a stream of its own beside other work,
//     it reports the clock that work runs at.
//   - The rate the scaled FP4 matrix cores sustain with nothing else to do: every wavefront
//     issues rounds of sixteen independent 32x32x64 products on codes taken from memory (so
//     their bits toggle like real operands), with no loads, LDS or barriers between them.
#include "kq_device.hpp"
#include "kq_launch.hpp"

namespace kq {

__global__ __launch_bounds__(64) void clock_probe_kernel(int64_t ticks, uint64_t* __restrict__ out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  while ((int64_t)(r - r0) < ticks) {
    __builtin_amdgcn_s_sleep(2);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r - r0;
  }
}

// Sixteen accumulators per wavefront (as many as a wavefront tile of the W4A4 GEMM), so that
// each product's issue never waits for a previous one's result; lane l's operands a and b are
// codes[l] and codes[64 + l] (16 bytes, 32 E2M1 codes each), the scales 2^0, and accumulator
// u takes (u & 1 ? a : b) times (u & 2 ? a : b).  Each wavefront stores one sum of its
// accumulators (so the products are not optimized away).
__global__ __launch_bounds__(256) void mfma_fp4_probe_kernel(int iters, const v4i* __restrict__ codes,
                                                             float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a4 = codes[lane], b4 = codes[64 + lane];
  const v8i a = v8i{a4.x, a4.y, a4.z, a4.w, 0, 0, 0, 0}, b = v8i{b4.x, b4.y, b4.z, b4.w, 0, 0, 0, 0};
  v16f acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 16; ++u)
      acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((u & 1) ? a : b, (u & 2) ? a : b, acc[u], 4, 4, 0, 127,
                                                               0, 127);
  }
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[u][e];
  sum = wave_sum(sum);
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = sum;
}

hipError_t launch_mfma_fp4_probe(int32_t iters, int32_t workgroups, const void* codes, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_fp4_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, (int)iters,
                     static_cast<const v4i*>(codes), out);
  return hipGetLastError();
}

hipError_t launch_clock_probe(int32_t spin_us, uint64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, (int64_t)spin_us * 100, out);
  return hipGetLastError();
}

}  // namespace kq
