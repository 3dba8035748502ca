/*
 * kq — the online 4-bit activation path of a quantized diffusion-transformer linear
 * layer, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The method (from the pages this library implements):
 *   - KroQuant (Kronecker-Structured Block Transforms for Efficient Post-Training
 *     Quantization of Diffusion Transformers), §01: Y = (XP)(P^-1 W) — an invertible
 *     transform P applied to the activations online, its inverse folded into the
 *     weights offline; §02: P = A (x) B (A 4x4, B 8x8) on every 32-element block of
 *     the activation vector; §03: 4-bit MXFP4 target format.
 *   - OrbitQuant (data-independent quantization for image and video DiTs), §03:
 *     RPBH(X) = X.P.H.D (random permutation, block Hadamard, random signs), the
 *     inverse folded offline as W' = R^-1 W, one Lloyd-Max codebook for all
 *     rotated coordinates.
 *   - CentriQ (Calibration-Free Quantization of DiTs via Exact Mean Centering),
 *     arXiv abstract: tokens are centred before the rotation and their means come
 *     back as a rank-1 fp16 term mu wbar^T; the per-token scale has a closed form.
 *   - SVDQuant explainer, §3: a 16-bit low-rank branch L1 L2 added to the 4-bit
 *     product, fused into the 4-bit kernel so it costs no separate pass; the branch
 *     holds the weight's leading singular directions, the residual is quantized.
 *   - DMQ explainer: channel-wise power-of-two scaling of outlier channels, a bit
 *     shift, as an optional step ahead of the transform.
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   X     fp16 [M][K]           activations, K a multiple of 32
 *   codes u8   [M][K/2]         two 4-bit codes per byte, element 2i in bits 0-3
 *   MXFP4 scales u8 [M][K/32]   E8M0 bytes (e + 127), one per 32 consecutive values
 *   LM4 scales  f32 [M]         per-token scale
 *   mu    fp16 [M]              per-token mean (centring)
 *   W     fp16 [K][N]           weights as in Y = X W (kq_fold_inverse_into_weights);
 *   Wt    fp16 [N][K]           the same weights in the [out][in] layout
 *                               (kq_fold_inverse_into_weights_nk, kq_svd_lowrank)
 *   wcodes u8 [N][K/2] (MXFP4) or [N][K/4] (2-bit, element 4i in bits 0-1)
 *   wscales u8 [N][K/32] (MXFP4) or fp16 [N][K/32] (2-bit group scales)
 *   wbar  fp16 [N]              column sums of W (rank-1 mean restore)
 *   L1    fp16 [r][K], L2 fp16 [N][r]   low-rank factors in the [out][in] layout
 *                               (X L1^T is the down-projection, T L2^T the up-projection:
 *                               the transposes of an L1 [K][r], L2 [r][N] written as
 *                               X L1 L2; rows are contiguous along the contracted
 *                               dimension, which is how the matrix cores take them)
 *   Y     fp16 [M][N]
 *
 * Ownership: the caller allocates and owns every buffer; the library never
 * allocates, frees or caches device memory, and holds no per-call state (it is
 * re-entrant).  Descriptor contents (kind, K, A, B) travel by value; perm, sign, P,
 * AB and pts are caller-owned device arrays.  Every call is asynchronous on `stream` (0 = the
 * null stream); inputs must stay alive until the stream has passed the call.
 *
 * Errors: the return value is a status.  Arguments are validated on the host
 * before anything is launched; a non-zero status means nothing was enqueued
 * (KQ_ERR_HIP: a launch itself failed, reported by hipGetLastError; in a call that
 * launches several kernels, those before the failing one may have been enqueued).  Faults
 * inside kernels surface at the caller's next synchronisation, as HIP defines.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KQ_ABI_VERSION 8

typedef int32_t kq_status;
enum {
  KQ_OK = 0,
  KQ_ERR_NULL = 1,         /* a required pointer is NULL */
  KQ_ERR_SHAPE = 2,        /* M, N < 1; K % 32 != 0; descriptor K != K; bad rank; mu without wbar */
  KQ_ERR_ALIGN = 3,        /* a device pointer is not 16-byte aligned */
  KQ_ERR_UNSUPPORTED = 4,  /* unknown enum, or a size outside the supported range */
  KQ_ERR_VALUE = 5,        /* a transform factor is singular or not finite */
  KQ_ERR_HIP = 6,          /* a HIP launch failed */
  KQ_ERR_WORKSPACE = 7     /* the workspace is missing or smaller than the call needs */
};

/* transform kinds */
enum { KQ_XFORM_NONE = 0, KQ_XFORM_KRON_4X8 = 1, KQ_XFORM_RPBH_32 = 2, KQ_XFORM_DENSE_32 = 3,
       KQ_XFORM_KRON_4X8_BLOCKS = 4 };
/* formats */
enum { KQ_FMT_MXFP4 = 0, KQ_FMT_LM4_TOKEN = 1, KQ_FMT_LM2_G32 = 2 };

/* One layer's block transform.
 * KRON_4X8 (KroQuant §02): every 32-element block x_b of a token is replaced by
 *   x_b . (A (x) B), i.e. with Xm[i][j] = x_b[8i+j]: Ym = A^T Xm B, y_b[8k+l] = Ym[k][l].
 *   A (4x4) and B (8x8) are row-major floats, one pair shared by all blocks.
 * RPBH_32 (OrbitQuant §03): y = x . Pi . blockdiag(H32) . D / sqrt(32) with
 *   (x.Pi)_j = x[perm[j]] over all K, H32 the Sylvester Hadamard matrix
 *   (H[i][j] = (-1)^popcount(i&j)), D = diag(sign), sign[j] in {-1, +1}.
 *   perm (int32 [K], a permutation of 0..K-1) and sign (int8 [K]) are device arrays,
 *   16- and 4-byte aligned.  perm is not checked on the device: an entry outside
 *   0..K-1 gives unspecified codes for that call (the on-chip gather cannot fault).
 * DENSE_32 (KroQuant §01, the block transform P before its Kronecker factorization):
 *   every 32-element block x_b is replaced by x_b . P, P a dense invertible 32x32 matrix
 *   (P: device float32 [32][32], row-major, 16-byte aligned; one P shared by all blocks).
 *   MXFP4 without centring only; the fold inverts P on the device (a singular P gives
 *   non-finite weights).
 * KRON_4X8_BLOCKS (KroQuant §02 with one factor pair per block index): block b of every
 *   token is replaced by x_b . (A_b (x) B_b), same convention as KRON_4X8, with
 *   AB: device float32 [K/32][80], 16-byte aligned; row b holds A_b (16, row-major) then
 *   B_b (64, row-major).  MXFP4 without centring only.  The factors are not checked: a
 *   non-finite entry gives unspecified codes, and the fold inverts each A_b (x) B_b on the
 *   device (a singular one gives non-finite weights for that block).
 * NONE: identity.
 * pts (optional, any kind but RPBH_32; DMQ explainer, channel-wise power-of-two scaling):
 *   device int8 [K], 16-byte aligned, entries e_k in 0..15.  The activation path first
 *   replaces x_k by fp16(x_k 2^-e_k) (round-to-nearest-even; exact unless the result is
 *   subnormal), then transforms; the fold multiplies weight input channel k by 2^e_k
 *   (exact) before the inverse transform, so the product is unchanged.  MXFP4 without
 *   centring only.  Entries are not checked on the device: one outside 0..15 gives
 *   unspecified codes for that call.  NULL: no scaling. */
typedef struct kq_xform {
  int32_t kind;
  int32_t reserved;          /* must be 0 */
  int64_t K;                 /* must equal the K of the call */
  float A[16];
  float B[64];
  const int32_t* perm;
  const int8_t* sign;
  const float* P;            /* DENSE_32 only */
  const float* AB;           /* KRON_4X8_BLOCKS only */
  const int8_t* pts;         /* NULL or per-channel power-of-two exponents */
} kq_xform;

/* KQ_ABI_VERSION of the built library. */
int32_t kq_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* kq_status_str(kq_status s);

/* Positive levels (ascending) of the symmetric n-level Lloyd-Max quantizer for a
 * unit Gaussian (OrbitQuant §03: one fixed codebook), as the library computes and
 * uses them; n = 4 or 16.  Host memory, n/2 doubles.  Runs on the host only. */
kq_status kq_lloyd_max_levels(int32_t n, double* levels_out);

/* Measurement helper, outside the activation path: the shader clock as the chip runs it
 * (the matrix-core peak scales with it), e.g. while other work occupies the GPU on another
 * stream.  One 64-thread workgroup on `stream` counts shader-clock cycles over spin_us
 * microseconds of the constant 100 MHz reference counter and writes the cycle count and
 * the reference ticks to out[0] and out[1] (device memory, caller-owned, 8-byte aligned);
 * the clock in MHz is 100 out[0] / out[1].  1 <= spin_us <= 1000000. */
kq_status kq_clock_probe(int32_t spin_us, uint64_t* out, hipStream_t stream);

/* Measurement helper, outside the activation path: the rate the scaled FP4 matrix cores
 * sustain with no memory traffic.  `workgroups` workgroups of four wavefronts on `stream`;
 * each wavefront issues `iters` rounds of sixteen independent v_mfma_scale_f32_32x32x64_f8f6f4
 * (E2M1 x E2M1, scales 2^0) on operands a, b read once from `codes` (device, 2048 bytes,
 * 16-byte aligned, caller-owned: lane l's a is bytes 16 l .. 16 l + 15, its b bytes 1024 + 16 l
 * .. ; product u of a round is (u & 1 ? a : b) x (u & 2 ? a : b)) and writes one sum of its
 * accumulators to out[4 * workgroup + wavefront] (device, 4 * workgroups floats,
 * caller-owned).  The work is 64 * iters * workgroups products of 2 * 32 * 32 * 64 flops; the
 * caller times the launch.  1 <= iters <= 1000000, 1 <= workgroups <= 65536. */
kq_status kq_mfma_fp4_probe(int32_t iters, int32_t workgroups, const void* codes, float* out, hipStream_t stream);

/* Online activation path (KroQuant §01-§03; OrbitQuant §03; CentriQ abstract):
 *   [centre]  mu_t = fp16(mean_k X[t,k]) (float32 sum), x <- x - mu_t      if center
 *   transform y = x . P  (xf->kind)
 *   quantize  fmt MXFP4: per 32-block a = max|y|, e = max(floor(log2 a) - 2, -127),
 *                        scale byte e + 127, code = E2M1 round-to-nearest-even of
 *                        y 2^-e, saturating at 6, sign bit = (y < 0); packed.
 *             fmt LM4_TOKEN: s_t = sqrt(mean_k y^2) (float32), code = sign-magnitude
 *                        index of y / s_t in the 16-level Lloyd-Max codebook
 *                        (a value on a threshold takes the smaller magnitude).
 * X fp16 [M][K]; codes u8 [M][K/2]; scales u8 [M][K/32] (MXFP4) or f32 [M] (LM4);
 * mu fp16 [M], required iff center != 0 (else ignored).
 * K % 32 == 0; K <= 16384 when centring, RPBH or LM4 is used (rows are staged on
 * chip).
 * All device pointers 16-byte aligned except mu and scales (4-byte for LM4). */
kq_status kq_transform_quantize(const kq_xform* xf, int32_t fmt, int32_t center,
                                const void* X, int64_t M, int64_t K,
                                uint8_t* codes, void* scales, void* mu,
                                hipStream_t stream);

/* Offline fold (KroQuant §01; OrbitQuant §03 W' = R^-1 W; CentriQ abstract):
 *   W' = P^-1 W (KRON: blockdiag(A^-1 (x) B^-1), the inverses computed on the host in
 *   double precision; RPBH: R^T; DENSE_32 / KRON_4X8_BLOCKS: inverted on the device),
 *   computed in float32 on the device, then each column n of W' (the weights of
 *   output n) quantized along K: fmt MXFP4 with the activation rule, or LM2_G32:
 *   s_g = fp16(RMS of the 32-group), 2-bit sign-magnitude code of w / s_g in the
 *   4-level Lloyd-Max codebook.  wbar[n] = fp16(sum_k W[k][n]) (float64 sum) if
 *   wbar != NULL: the column sums for the rank-1 mean restore.
 * W fp16 [K][N] (row-major: W[k][n] at k*N + n); wcodes u8 [N][K/2] (MXFP4) or [N][K/4]
 * (LM2); wscales u8 [N][K/32] (MXFP4) or fp16 [N][K/32] (LM2); wbar fp16 [N].
 * Untimed: runs once per layer.  Returns KQ_ERR_VALUE if A or B is singular. */
kq_status kq_fold_inverse_into_weights(const kq_xform* xf, int32_t fmt,
                                       const void* W, int64_t K, int64_t N,
                                       uint8_t* wcodes, void* wscales, void* wbar,
                                       hipStream_t stream);

/* The same fold for weights given as Wt fp16 [N][K] (the [out][in] layout, Wt[n][k] =
 * W[k][n]); outputs identical to kq_fold_inverse_into_weights on the same weights. */
kq_status kq_fold_inverse_into_weights_nk(const kq_xform* xf, int32_t fmt,
                                          const void* Wt, int64_t N, int64_t K,
                                          uint8_t* wcodes, void* wscales, void* wbar,
                                          hipStream_t stream);

/* Low-rank down-projection of the 16-bit branch (SVDQuant explainer §3):
 *   T = fp16(X L1^T), fp32 accumulation on the fp16 matrix cores.
 * X fp16 [M][K] (the original activations: not centred, not transformed), L1 fp16 [r][K],
 * T fp16 [M][r] (caller-owned).  r in {16, 32, 48, 64}; K % 32 == 0, K <= 2^20.
 * workspace (optional, caller-owned device memory, 16-byte aligned): when M is small
 *   against the device, K is split over several workgroups whose fp32 partials go to the
 *   workspace, and a second kernel sums them in a fixed order (results do not depend on
 *   scheduling).  kq_lowrank_down_workspace_bytes gives the size that enables the full
 *   split; a smaller workspace gives fewer slices, and NULL / 0 runs unsplit (same
 *   results up to fp32 summation order, slower for small M).  The library allocates
 *   nothing.  Calls that share a workspace must not overlap. */
size_t kq_lowrank_down_workspace_bytes(int64_t M, int64_t K, int32_t r);
kq_status kq_lowrank_down(const void* X, const void* L1, int64_t M, int64_t K, int32_t r,
                          void* T, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The online activation path and the low-rank down-projection in one pass over X
 * (SVDQuant explainer §3: the 16-bit branch and the 4-bit branch read the same input, and
 * running the branch separately costs an extra read of it):
 *   codes, scales[, mu] = MXFP4 of the (optionally centred) block-transformed X, as
 *                   kq_transform_quantize with fmt MXFP4;
 *   T = fp16(X L1^T) from the original X (neither centred nor transformed), as
 *                   kq_lowrank_down.
 * Kinds NONE, KRON_4X8 and DENSE_32 (no centring): one kernel, X read once.  RPBH_32
 * (centring optional; mu fp16 [M], required iff center != 0): the permutation spans the
 * whole row, so the call runs the row-staged transform and then the down-projection
 * (X is read twice; results equal those of the two separate calls).  No pts.
 * Shapes, layouts, alignment and the workspace rule are those of the two calls it
 * replaces; kq_lowrank_down_workspace_bytes(M, K, r) gives the workspace size.  For the
 * one-kernel kinds, codes may differ from kq_transform_quantize's only at rounding ties of
 * the float32 arithmetic, and T from kq_lowrank_down's only by float32 summation order. */
kq_status kq_transform_quantize_lowrank(const kq_xform* xf, int32_t center, const void* X, int64_t M, int64_t K,
                                        uint8_t* codes, void* scales, void* mu, const void* L1, int32_t r, void* T,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Offline rank-r extraction of the 16-bit branch (SVDQuant explainer §3: the weight's
 * leading singular directions stay in 16 bits, the residual is quantized to 4 bits):
 *   W (fp16 [N][K], row n = output n) ~ L2 L1 with L2 = U_r S_r^1/2 (fp16 [N][r]),
 *   L1 = S_r^1/2 V_r^T (fp16 [r][K]) from the r leading singular triplets, and
 *   R = fp16(W - L2 L1) (fp16 [N][K]) computed with the fp16 factors, to be folded and
 *   quantized in place of W (kq_fold_inverse_into_weights; its wbar is then 1^T R).
 *   sigma (optional, float [r]): the singular value estimates, descending.
 * The subspace comes from randomized subspace iteration (Halko, Martinsson and Tropp 2011,
 * algorithms 4.4 / 5.1) started from the caller's omega (float32 [K][l], e.g. Gaussian;
 * the library draws no random numbers) with l - r extra columns and `iters` power steps,
 * re-orthonormalized after every product; float32 products, float64 for the l x l parts.
 * Accuracy depends on the gap between sigma_r and sigma_{l+1} and on iters.
 * r in {16, 32, 64}; r < l <= 96, l <= min(N, K); 0 <= iters <= 16; K % 32 == 0.
 * workspace: caller-owned device memory of kq_svd_lowrank_workspace_bytes(N, K, r, l)
 * bytes, 256-byte aligned; other pointers 16-byte aligned (sigma 4).  Runs several kernels
 * on `stream`; calls sharing a workspace must not overlap. */
size_t kq_svd_lowrank_workspace_bytes(int64_t N, int64_t K, int32_t r, int32_t l);
kq_status kq_svd_lowrank(const void* W, int64_t N, int64_t K, int32_t r, const float* omega, int32_t l,
                         int32_t iters, void* L1, void* L2, void* R, float* sigma, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* The 4-bit linear with its full-precision branches (KroQuant §01: Y = (XP)(P^-1 W);
 * SVDQuant explainer §3: plus the 16-bit low-rank branch X L1 L2; CentriQ abstract: plus
 * the rank-1 mean restore):
 *   Y = Xq . Wq^T  +  (X L1^T) L2^T  +  mu wbar^T          (fp32 accumulate, fp16 out)
 * fmt MXFP4: Xq, Wq MXFP4 (xscales u8 [M][K/32], wscales u8 [N][K/32]); products on
 *   the scaled-FP4 matrix cores, each block pair scaled by 2^(ex+ew).  K % 128 == 0.
 * fmt LM2_G32 (W2A4): Xq per-token Lloyd-Max 4-bit (xscales f32 [M]), Wq 2-bit groups
 *   (wcodes u8 [N][K/4], wscales fp16 [N][K/32]); the codebooks are the library's own
 *   (kq_lloyd_max_levels).  K % 32 == 0.  No low-rank or rank-1 branch (r must be 0).
 * Low-rank branch: X fp16 [M][K] (the original activations, neither centred nor
 *   transformed), L1 fp16 [r][K], L2 fp16 [N][r], r in {0, 16, 32, 48, 64} (0: X, L1,
 *   L2 ignored and may be NULL).  The down-projection T = X L1^T runs first on the
 *   stream (as kq_lowrank_down, T held in the workspace), then one GEMM kernel whose
 *   accumulators start from T L2^T, so the branch adds no pass over Y.
 *   T is rounded to fp16 (the up-projection is an fp16 matrix-core product; the
 *   explainer keeps the branch in 16 bits): the branch then carries a relative error
 *   of at most 2^-11 per T entry, far below the 4-bit product's.
 * Rank-1 restore: mu fp16 [M] and wbar fp16 [N], both or neither.
 * workspace: caller-owned device memory, 256-byte aligned, of at least
 *   kq_w4a4_linear_workspace_bytes(M, r) bytes (0 when r == 0; NULL allowed then).  It
 *   holds T and the split-K partial sums of the down-projection.  The library
 *   allocates nothing.  Calls that share a workspace must not overlap.
 * N % 16 == 0; M <= 2^30, N and K <= 2^20.  Y fp16 [M][N].  Pointers 16-byte aligned,
 *   except xscales and wscales (4) and mu (2).
 * Errors: KQ_ERR_WORKSPACE if r > 0 and the workspace is NULL or too small. */
size_t kq_w4a4_linear_workspace_bytes(int64_t M, int32_t r);
kq_status kq_w4a4_linear(int32_t fmt,
                         const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                         const uint8_t* wcodes, const void* wscales, int64_t N,
                         const void* X, const void* L1, const void* L2, int32_t r,
                         const void* mu, const void* wbar,
                         void* Y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): kq_w4a4_linear without a workspace argument.  T and the
 * down-projection's split-K partial sums live in a fixed device array of
 * KQ_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the process ends);
 * the call allocates nothing and calls no allocating routine.  Rejected with
 * KQ_ERR_WORKSPACE when T alone (M * r * 2 bytes, rounded up to 256) exceeds that size;
 * when T fits but the partial sums of the full split do not, fewer K slices are used
 * (results then differ from kq_w4a4_linear's only in float32 summation order).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and give undefined results.  Arguments otherwise as
 * kq_w4a4_linear. */
#define KQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
kq_status kq_w4a4_linear_noalloc(int32_t fmt,
                                 const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                                 const uint8_t* wcodes, const void* wscales, int64_t N,
                                 const void* X, const void* L1, const void* L2, int32_t r,
                                 const void* mu, const void* wbar,
                                 void* Y, hipStream_t stream);

/* The same linear with the down-projection already done: T fp16 [M][r] from
 * kq_lowrank_down or kq_transform_quantize_lowrank (caller-owned), L2 fp16 [N][r],
 * r in {0, 16, 32, 48, 64} (0: T and L2 ignored).  One kernel launch; no workspace.
 * Other arguments and rules as kq_w4a4_linear. */
kq_status kq_w4a4_linear_t(int32_t fmt,
                           const uint8_t* xcodes, const void* xscales, int64_t M, int64_t K,
                           const uint8_t* wcodes, const void* wscales, int64_t N,
                           const void* T, const void* L2, int32_t r,
                           const void* mu, const void* wbar,
                           void* Y, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KQ_H */
