// Device-side helpers shared by the kq kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));   // 16 raw bytes (a native vector: copies stay in registers)

// DPP quad_perm control word: lane i of each quad reads lane sel[i] of the same quad.
constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Value of lane I of this lane's quad.
template <int I>
__device__ __forceinline__ float quad_bcast(float v) { return dpp_f<quad_perm(I, I, I, I)>(v); }

// Value of the lane whose quad index differs in bit 0 / bit 1.
__device__ __forceinline__ float quad_xor1(float v) { return dpp_f<quad_perm(1, 0, 3, 2)>(v); }
__device__ __forceinline__ float quad_xor2(float v) { return dpp_f<quad_perm(2, 3, 0, 1)>(v); }

// Sum over the 16 lanes of a DPP row (every lane of the row gets the result): rotations
// by 8 and 4 within the row, then the two quad exchanges.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);   // row_ror:8
  v += dpp_f<0x124>(v);   // row_ror:4
  v += quad_xor2(v);
  v += quad_xor1(v);
  return v;
}

// Max over the four lanes of a quad (every lane gets the result).
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, quad_xor1(v));
  return fmaxf(v, quad_xor2(v));
}

// E8M0 shared-scale byte of a block from its largest magnitude a >= 0 (OCP MX rule):
// e = floor(log2 a) - 2 clamped below at -127, stored as e + 127.  For a normal float
// floor(log2 a) is its exponent field minus 127; a zero or subnormal a (exponent field
// 0, i.e. a < 2^-126) gives e < -127, which clamps to byte 0.
__device__ __forceinline__ uint32_t e8m0_byte(float a) {
  uint32_t ef = (__float_as_uint(a) >> 23) & 0xFFu;
  return ef > 2u ? ef - 2u : 0u;
}

// The conversion scale 2^e as the float whose exponent field is the E8M0 byte.  The
// gfx950 packed FP4 conversion divides by 2^(exponent field - 127) and ignores the
// mantissa; exponent field 0 stands for 2^-127.
__device__ __forceinline__ float e8m0_as_cvt_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// Eight fp32 values -> eight E2M1 codes (round to nearest even, saturating at 6),
// element 2i in the low nibble of byte i.  Inputs must not be -0.0 (the hardware keeps
// the sign of a negative zero; the format contract maps exact zeros to code 0).
__device__ __forceinline__ uint32_t cvt8_fp4(const float* y, float scale) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
  return w;
}

__device__ __forceinline__ void unpack8_f16(const uint4& raw, float* x) {
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 f = __half22float2(h[i]);
    x[2 * i] = f.x;
    x[2 * i + 1] = f.y;
  }
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it does not
// wait for this wave's outstanding global loads, so prefetches stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void unpack8_f16(const v4u& raw, float* x) {
  const v8h h = __builtin_bit_cast(v8h, raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}

// acc + (lo half + hi half) of a packed fp16 pair, in fp32 (the products by 1 are exact).
// The pair is taken by value: a bit cast applied directly to an element of a vector
// variable has been seen to read element 0 for every index.
__device__ __forceinline__ float add_f16x2(uint32_t pair, float acc) {
  typedef __fp16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pair), (h2){1.0f, 1.0f}, acc, false);
}

// acc + a.x^2 + a.y^2 for a pair of halves (exact products, float32 accumulation).
__device__ __forceinline__ float sq_f16x2(uint32_t pair, float acc) {
  typedef __fp16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = __builtin_bit_cast(h2, pair);
  return __builtin_amdgcn_fdot2(v, v, acc, false);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros and stores
// past the end are dropped, which handles ragged tiles and masked lanes without branches
// (a masked lane uses an offset of at least KQ_OOB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
#define KQ_OOB 0x7FFFFFF0

// ---- loads from global memory straight into LDS (buffer loads with the LDS destination)
typedef int v4i __attribute__((ext_vector_type(4)));

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations
// of this wave are outstanding and does not wait on the other counters.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Buffer resource words for [base, base + bytes) (raw buffer, no stride, as make_rsrc).
__device__ __forceinline__ v4i rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)(bytes < 0 ? 0 : bytes);
  return v4i{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), n, 0x00020000};
}
// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 64 lanes x 16 bytes from rsrc at byte offset voff (per lane, range-checked) into LDS
// at lds + 16 x lane.  The LDS address must be wave-uniform (it goes to M0): it is passed
// through readfirstlane so that it lives in a scalar register.
__device__ __forceinline__ void lds_load16(const v4i& rsrc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// Sum over a wavefront (every lane gets the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace kq
