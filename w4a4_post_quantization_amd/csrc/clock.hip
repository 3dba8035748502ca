// Measurement helper: the shader clock as the chip runs it.  One wavefront counts
// shader-clock cycles (s_memtime) against the constant 100 MHz reference counter
// (s_memrealtime) for a requested span of reference time; launched on a stream of its own
// beside other work, it reports the clock that work runs at.
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

hipError_t launch_clock_probe(int32_t spin_us, uint64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, (int64_t)spin_us * 100, out);
  return hipGetLastError();
}

}  // namespace kq
