// Host-side launchers of the kq kernels (internal to the library; the C ABI in kq.h
// validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kq {

struct KronFactors {
  float A[16];  // row-major 4x4
  float B[64];  // row-major 8x8
};

// Lloyd-Max codebooks for a unit Gaussian, as float32 for the kernels.
struct LmTables {
  float t16[7];   // positive thresholds of the 16-level quantizer (ascending)
  float l16[8];   // positive levels of the 16-level quantizer
  float t4;       // positive threshold of the 4-level quantizer
  float l4[2];    // positive levels of the 4-level quantizer
};
const LmTables& lm_tables();
bool lloyd_max_levels(int n, double* out);


// Matrix-core block transforms + MXFP4: streaming identity (kind 0), Kronecker (1) or
// dense 32x32 P (3, device, row-major) without centring, and row-staged RPBH with
// optional centring.
// Per-block Kronecker factors AB (device float [K/32][80]: A then B, row-major, per block
// index) + MXFP4 for X [M][K]; pts optional as below.
hipError_t launch_kron_blocks_mx(const __half* X, int64_t M, int64_t K, const float* AB, const int8_t* pts,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s);
// pts (optional, device int8 [nbk * 32]): per-channel power-of-two exponents applied first.
hipError_t launch_kron_mx_mfma(int kind, const __half* X, int64_t nblocks, const KronFactors& f, const float* P,
                               const int8_t* pts, int64_t nbk, uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_rpbh_mx_mfma(bool center, const __half* X, int64_t M, int64_t K, const int32_t* perm,
                               const int8_t* sign, uint8_t* codes, uint8_t* scales, __half* mu, hipStream_t s);
// RPBH + per-token Lloyd-Max 4-bit codes (no centring) on the row-group kernel: codes
// [M][K/2], scales float [M] (s_t = ||x_t|| / sqrt(K)).
hipError_t launch_rpbh_lm4_mfma(const __half* X, int64_t M, int64_t K, const int32_t* perm, const int8_t* sign,
                                uint8_t* codes, float* scales, hipStream_t s);

// Row-staged transform + quantize: any transform, optional centring, MXFP4 or LM4.
// kind: 0 none, 1 kron, 2 rpbh; fmt: 0 MXFP4, 1 LM4.
hipError_t launch_row_quant(int kind, int fmt, bool center, const __half* X, int64_t M, int64_t K,
                            const KronFactors& f, const int32_t* perm, const int8_t* sign,
                            uint8_t* codes, void* scales, __half* mu, hipStream_t s);

// Offline fold: W'^T rows = inverse transform of W^T rows, quantized along K.
// fmt: 0 MXFP4, 2 LM2.  f holds the INVERSE factors for kind 1.
// kind 3: P (device, row-major) is inverted on the device; kind 4: P is the per-block
// factor table (float [K/32][80]) and each block's A (x) B is inverted on the device.  pts (optional): weight input
// channel k is multiplied by 2^pts[k] before the inverse transform.
// kn: W is [K][N] (element (n, k) at k * N + n); else [N][K] (at n * K + k).
hipError_t launch_fold(int kind, int fmt, bool kn, const __half* W, int64_t N, int64_t K, const KronFactors& finv,
                       const int32_t* perm, const int8_t* sign, const float* P, const int8_t* pts, uint8_t* wcodes,
                       void* wscales, hipStream_t s);
// wbar[n] = fp16(sum_k W(n, k)), summed in float64; layout as launch_fold.
hipError_t launch_colsum(bool kn, const __half* W, int64_t N, int64_t K, __half* wbar, hipStream_t s);

// T[M][r] = fp16(X L1^T), fp32 accumulation; split over K into `part` (fp32 partials,
// part_bytes long, may be null) when that helps and fits.
size_t lowrank_workspace_bytes(int64_t M, int64_t K, int r);
// The linear's workspace: T fp16 [M][r] (lowrank_t_bytes, 256-byte padded) then split-K
// partials for any K.
size_t lowrank_t_bytes(int64_t M, int r);
size_t lowrank_linear_workspace_bytes(int64_t M, int r);
hipError_t launch_lowrank_down(const __half* X, const __half* L1, int64_t M, int64_t K, int r,
                               __half* T, float* part, size_t part_bytes, hipStream_t s);
// The same down-projection fused with the block transform (kind 0 identity, 1 Kronecker,
// 3 dense P) and MXFP4 of X (codes [M][K/2], scales [M][K/32]): X is read once.
hipError_t launch_lowrank_xform_mx(int kind, const __half* X, const __half* L1, int64_t M, int64_t K, int r,
                                   __half* T, float* part, size_t part_bytes, const KronFactors& fk, const float* P,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s);

// Y = Xq Wq^T (+ T L2^T) (+ mu wbar^T), MXFP4 x MXFP4.
// Offline rank-r extraction: Wt [N][K] fp16 -> L1 [r][K], L2 [N][r], R = fp16(Wt - L2 L1)
// [N][K] (fp16), sigma [r] (optional); omega [K][l] float32 starting block; workspace of
// svd_workspace_bytes(N, K, l, r) bytes, 256-byte aligned.
size_t svd_workspace_bytes(int64_t N, int64_t K, int l, int r);
hipError_t launch_svd_lowrank(const __half* Wt, int64_t N, int64_t K, int r, const float* omega, int l, int iters,
                              __half* L1, __half* L2, __half* R, float* sigma, void* workspace, hipStream_t s);

hipError_t launch_w4a4_gemm(const uint8_t* xcodes, const uint8_t* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const uint8_t* wscales, int64_t N,
                            const __half* T, const __half* L2, int r, const __half* mu,
                            const __half* wbar, __half* Y, hipStream_t s);

// Y = (s_t l16[qx]) (s_g l4[qw])^T, per-token Lloyd-Max activations x 2-bit weights.
hipError_t launch_w2a4_gemm(const uint8_t* xcodes, const float* xscales, int64_t M, int64_t K,
                            const uint8_t* wcodes, const __half* wscales, int64_t N, __half* Y,
                            hipStream_t s);

int device_cu_count();
// Workgroups of `kernel` that can be resident on one compute unit at once.
// Shader-clock cycles and 100 MHz reference ticks over spin_us microseconds (out: device
// uint64 [2]); one 64-thread workgroup.
hipError_t launch_clock_probe(int32_t spin_us, uint64_t* out, hipStream_t s);
hipError_t launch_mfma_fp4_probe(int32_t iters, int32_t workgroups, const void* codes, float* out, hipStream_t s);

int resident_blocks_per_cu(const void* kernel, int threads, size_t lds);

}  // namespace kq
