/*
 * svdq.h — C ABI of the SVDQuant linear operator for AMD Instinct MI355X (gfx950).
 *
 *   Y = (X^ L1) L2 + Q(X^) Q(R),   X^ = x / scale,   L1 L2 = rank-r truncated SVD of
 *   scale[:,None] * W,   R = scale[:,None] * W - L1 L2.
 *
 * Sources, cited by page title and section:
 *   [EX]  "SVDQuant Smoothing, Low-rank and Residual Quantization" (paperleet exercise):
 *         "Functions / Return requirements" (smooth_inputs, split_weight, svdquant_linear,
 *         fake_quantize, _check_smoothing, _check_rank) and "Formula and conventions" items 1-3.
 *   [FI]  "flashinfer.gemm.svdquant_linear" (API page): the three-step chain (smooth+quantise,
 *         down-projection GEMM, residual GEMM with low-rank epilogue), offline preparation by
 *         the caller, rank a multiple of 32.
 *   [MS]  "SVDQuant 参数配置流程指南" (msModelSlim usage guide), step 2: MXFP4 per-block
 *         symmetric minmax quantisation of activations and weights, rank 32.
 *
 * Conventions for every call
 *   - Layout: x is [B, M], weight is [M, N] (not the transposed Linear layout), scale is [M],
 *     Y is [B, N]. Matrices are row-major with an explicit row stride in ELEMENTS; the
 *     elementwise calls also take a column stride (strided inputs, [EX] "Formula and
 *     conventions", last paragraph).
 *   - dtype: SVDQ_F32 or SVDQ_BF16 for x, weight and every dtype-typed output (they share one
 *     dtype); scale is always float32. float64 is rejected with SVDQ_EDTYPE.
 *   - Ownership: the caller owns every buffer (inputs, outputs, prepared weights, workspace).
 *     The library never allocates device memory and never writes an input. Outputs must not
 *     overlap inputs.
 *   - Device calls take a hipStream_t, only enqueue work on it (asynchronous, stream-ordered)
 *     and return; faults inside kernels surface at the caller's next synchronisation.
 *   - Errors: every call returns an svdq_status; svdq_last_error() gives a message for the
 *     last failing call on the calling thread. Invalid arguments ([EX] _check_smoothing,
 *     _check_rank, 2 <= bits <= 8) return SVDQ_EINVAL before any work is enqueued.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* svdq_stream_t; /* the same handle as hipStream_t */

typedef enum {
  SVDQ_OK = 0,
  SVDQ_EINVAL = 1,       /* invalid shape, stride, rank, bits, scale or buffer size */
  SVDQ_EDTYPE = 2,       /* unsupported dtype (e.g. float64) */
  SVDQ_EUNSUPPORTED = 3, /* a valid request this library does not implement */
  SVDQ_EHIP = 4          /* a HIP runtime call failed (launch error, bad device pointer) */
} svdq_status;

typedef enum { SVDQ_F32 = 0, SVDQ_BF16 = 1, SVDQ_F64 = 2 } svdq_dtype;

typedef enum {
  SVDQ_FMT_INT = 0, /* per-tensor symmetric INT, 2 <= bits <= 8 ([EX] fake_quantize rule) */
  SVDQ_FMT_MX = 1   /* MXFP4: E2M1 codes, one E8M0 scale per 32 elements along K ([MS] step 2) */
} svdq_format;

/* Message of the last failing call on this thread ("" if none). Never NULL. */
const char* svdq_last_error(void);

/* Library version string, e.g. "svdq 0.1 gfx950". */
const char* svdq_version(void);

/* --------------------------------------------------------------------------------------
 * svdq_smooth_inputs — [EX] smooth_inputs / "Formula and conventions" item 1.
 *   xs[b,m] = D(x[b,m] / scale[m]),  ws[m,n] = D(scale[m] * weight[m,n]),
 * with IEEE binary32 division / multiplication and D = rounding to dtype (RNE for bf16).
 * xs @ ws equals x @ weight up to that rounding. Device pointers.
 *   x: [B,M] with strides (sxb, sxm); weight: [M,N] with strides (swm, swn); scale: [M] f32,
 *   contiguous. xs_out: [B,M] row stride ldxs (unit column stride); ws_out: [M,N] row
 *   stride ldws. Either of (x, xs_out) or (weight, ws_out) may be NULL to skip that half.
 * Errors: EINVAL (empty, bad stride), EDTYPE. Scale positivity is the caller's contract
 *   on the device path (checking it would need a device read); svdq_check_smoothing
 *   validates a host copy.
 * ------------------------------------------------------------------------------------ */
int svdq_smooth_inputs(const void* x, int64_t B, int64_t M, int64_t sxb, int64_t sxm,
                       const void* weight, int64_t N, int64_t swm, int64_t swn,
                       const float* scale, int dtype,
                       void* xs_out, int64_t ldxs, void* ws_out, int64_t ldws,
                       svdq_stream_t stream);

/* --------------------------------------------------------------------------------------
 * svdq_check_smoothing / svdq_check_rank — [EX] _check_smoothing and _check_rank on host
 * data: B, M, N >= 1, every scale[m] positive and finite, 0 <= rank <= min(M,N).
 * Return SVDQ_OK or SVDQ_EINVAL with a message.
 * ------------------------------------------------------------------------------------ */
int svdq_check_smoothing(int64_t B, int64_t M, int64_t Mw, int64_t Ms, int64_t N, const float* scale_host);
int svdq_check_rank(int64_t M, int64_t N, int64_t rank);

/* --------------------------------------------------------------------------------------
 * svdq_split_weight — [EX] split_weight / "Formula and conventions" item 2. HOST call.
 * Truncated SVD of weight [M,N] (host, row stride ldw, dtype) computed in float64 by the
 * library (one-sided Jacobi for small matrices, randomized subspace iteration with a
 * Rayleigh-Ritz step for large ones; no LAPACK):
 *   left  = D(U_r diag(sigma_r))  [M, r] row-major contiguous,
 *   right = D(V_r^T)              [r, N] row-major contiguous,
 *   residual = D(weight - left @ right) [M, N] row-major contiguous, the product taken in
 *   float64 from the stored (rounded) factors.
 * rank 0 writes nothing to left/right (they may be NULL) and copies weight to residual.
 * Singular-vector signs are free; the result is deterministic for a given input.
 * Errors: EINVAL (rank out of [0, min(M,N)], empty), EDTYPE.
 * ------------------------------------------------------------------------------------ */
int svdq_split_weight(const void* weight, int64_t M, int64_t N, int64_t ldw, int dtype, int64_t rank,
                      void* left, void* right, void* residual);

/* --------------------------------------------------------------------------------------
 * svdq_fake_quantize — [EX] fake_quantize / "Formula and conventions" item 3. Device call.
 * One scale per tensor: qmax = 2^(bits-1)-1, s = max|z| / qmax (binary32 division),
 * out = D(s * clamp(round_half_even(z / s), -qmax, qmax)); an all-zero tensor gives zeros.
 *   z: [rows, cols] with strides (szr, szc); out: [rows, cols] row stride ldo.
 *   workspace: device scratch of at least svdq_fake_quantize_workspace(rows, cols) bytes
 *   (per-block partial maxima; no initialisation needed).
 *   s_out: optional device float* receiving s (may be NULL).
 * Errors: EINVAL (bits outside [2,8], empty, workspace too small), EDTYPE.
 * ------------------------------------------------------------------------------------ */
size_t svdq_fake_quantize_workspace(int64_t rows, int64_t cols);
int svdq_fake_quantize(const void* z, int64_t rows, int64_t cols, int64_t szr, int64_t szc, int dtype,
                       int bits, void* out, int64_t ldo, float* s_out,
                       void* workspace, size_t workspace_bytes, svdq_stream_t stream);

/* --------------------------------------------------------------------------------------
 * Prepared weights ([FI]: the per-layer invariants are prepared offline by the caller).
 * One contiguous blob, built on the host by svdq_prepare, copied to the device by the
 * caller, and passed to svdq_linear. Sections (byte offsets from svdq_prepared_layout,
 * each 256-byte aligned), with Kp = M rounded up to 256, Np = N rounded up to 256 and
 * rp = rank rounded up to 32 (zero padding is exact: padded codes and factors are 0):
 *   SVDQ_SEC_SCALE   float32 [M]       the smoothing scale (divisor of x)
 *   SVDQ_SEC_RCODES  R^T codes, two 4-bit codes per byte with even k in the low nibble
 *                    (MX: E2M1; INT bits<=4: two's-complement nibbles), or int8 for INT
 *                    bits>4. INT: [Np, Kp/2] (or [Np, Kp]) bytes, K-contiguous per output
 *                    column n. MX: Np * Kp/2 bytes in 1 KB tiles, byte j (codes 2j, 2j+1)
 *                    of column n at ((n/16) * (Kp/128) + j/64) * 1024 + (n%16) * 64 + j%64
 *                    (each 16-column x 128-code block is contiguous: one wave-wide load)
 *   SVDQ_SEC_RSCALES MX: Np * Kp/32 E8M0 bytes (e + 127), one per 32-block of column n,
 *                    stage-tiled: the byte of (n, block kb) sits at
 *                    ((n/64) * (Kp/128) + kb/4) * 256 + (n%64) * 4 + kb%4
 *                    (a 128-code stage's scales for 64 columns are 256 contiguous bytes);
 *                    INT: one float32 s_R
 *   SVDQ_SEC_L1T     dtype, rp * Kp    L1^T (down-projection factor, transposed), tiled for
 *                    the matrix cores: with E = 16 / sizeof(dtype) elements per 16 bytes,
 *                    element (t, k) sits at ((t/16) * (Kp/128) + k/128) * 2048
 *                    + ((((k%32)/E) * 4 + (k%128)/32) * 16 + t%16) * E + k%E
 *                    (each 16-row x 128-K tile is 2048 contiguous elements, ordered so one
 *                    wave reads a K-slice of it with one 1 KB request)
 *   SVDQ_SEC_L2T     dtype [Np, rp]    L2^T (up-projection factor, transposed)
 *   SVDQ_SEC_RECIP   float32 [M]       RN(1/scale[m]), or 0 where scale[m] lies outside
 *                    [2^-90, 2^90]; the kernels use it for an exact fast x / scale
 *   SVDQ_SEC_GLOBAL  float32 [4]       MX two-level scaling (svdq_prepare_two_level):
 *                    {g_x, g_R, alpha, 0}, the activation and residual global scales and
 *                    alpha = RN(1 / (g_x g_R)); {1, 1, 1, 0} for every other preparation
 * ------------------------------------------------------------------------------------ */
enum {
  SVDQ_SEC_SCALE = 0,
  SVDQ_SEC_RCODES = 1,
  SVDQ_SEC_RSCALES = 2,
  SVDQ_SEC_L1T = 3,
  SVDQ_SEC_L2T = 4,
  SVDQ_SEC_RECIP = 5,
  SVDQ_SEC_GLOBAL = 6,
  SVDQ_SEC_END = 7, /* offsets[SVDQ_SEC_END] = total blob bytes */
  SVDQ_NSEC = 8
};

/* Offsets of every section and the total size. Errors: EINVAL, EDTYPE, EUNSUPPORTED (INT
 * formats whose residual products could leave int32: (M rounded up to 256) * qmax^2 * (256
 * for bits <= 4, else 1) must be below 2^31, e.g. M <= 171008 at 4 bits, M <= 133120 at 8;
 * the same rule holds for the svdq_prepare* calls and svdq_linear*). */
int svdq_prepared_layout(int64_t M, int64_t N, int64_t rank, int fmt, int bits, int dtype,
                         int64_t offsets[SVDQ_NSEC]);

/* --------------------------------------------------------------------------------------
 * svdq_prepare — one-time HOST preparation ([EX] svdquant_linear: smooth, then split the
 * smoothed weight, quantise the residual; [MS] iter_smooth -> svd_res -> linear_quant):
 *   ws = D(scale[:,None] * weight)  (binary32 product, rounded to dtype)
 *   (left, right, residual) = svdq_split_weight(ws, rank)
 *   residual quantised per tensor (INT: s_R = max|R|/qmax, codes) or per 32-block along M
 *   for each column n (MX), then packed into the blob layout above.
 *   weight [M,N] host row stride ldw, scale [M] host float32, blob_host of
 *   offsets[SVDQ_SEC_END] bytes. left_out [M,rank], right_out [rank,N], residual_out [M,N]
 *   (host, dtype, contiguous) optionally receive the exact factors and R used (may be NULL).
 * Errors: EINVAL ([EX] _check_smoothing/_check_rank cases, bits, MX with bits != 4), EDTYPE.
 * ------------------------------------------------------------------------------------ */
int svdq_prepare(const void* weight, int64_t M, int64_t N, int64_t ldw, const float* scale,
                 int64_t rank, int fmt, int bits, int dtype, void* blob_host,
                 void* left_out, void* right_out, void* residual_out);
/* The same preparation with the truncated SVD on the GPU: the randomized subspace iteration
 * (k = rank + 32 panel columns, 16 power iterations) and its Rayleigh-Ritz step run in float64 on
 * the device — panel products with the smoothed weight on float64 matrix cores, the panels
 * orthonormalised by Cholesky-QR twice (the k x k Cholesky factorisations on the host), the
 * Rayleigh-Ritz one-sided Jacobi on the device; the fold, the residual and the quantisation stay
 * on the host. The result satisfies the same contract (a best rank-r approximation up to the
 * randomized route's accuracy) but is not bit-identical to svdq_prepare's. Matrices with
 * min(M, N) <= 512, or with rank + 32 above 256 panel columns, take the host's split and need no
 * workspace. workspace: device, 256-byte aligned, >= svdq_prepare_gpu_workspace_bytes bytes
 * (the float32 weight, three float64 panels of max(M, N) x k, a k x N float64 projection and
 * k x k matrices); the call enqueues copies and kernels on `stream` and waits for them (host
 * call). Errors as svdq_prepare, plus EINVAL for a small workspace and EHIP. */
int svdq_prepare_gpu_workspace_bytes(int64_t M, int64_t N, int64_t rank, size_t* bytes_out);
int svdq_prepare_gpu(const void* weight, int64_t M, int64_t N, int64_t ldw, const float* scale,
                     int64_t rank, int fmt, int bits, int dtype, void* blob_host,
                     void* left_out, void* right_out, void* residual_out,
                     void* workspace, size_t workspace_bytes, svdq_stream_t stream);

/* MXFP4 with two-level scaling ([FI] svdquant_linear: an activation global scale and a
 * per-tensor residual scale alpha over the block scales, with the low-rank up-projection
 * factor prepared divided by alpha, [FI]'s l1_scaled, so that the epilogue applies alpha
 * once; that factor is L2 in this library's notation): the residual is quantised
 * as z_R = RN(R * g_R), E8M0 per 32-block of z_R, where g_R = RN(6 * 2^ex / max|R|) with
 * max|R| / 6 = f * 2^ex, f in [0.5, 1) (so g_R lies in (1, 2] and the largest |z_R| is 6 * 2^ex
 * up to rounding; g_R = 1 for an all-zero R); each call quantises the activations as
 * z_x = RN(X^ * g_x) with the caller's x_global_scale g_x (finite, in [2^-64, 2^64]; a value
 * calibrated offline, as the residual's; every product RN(X^ * g_x) must stay finite, an
 * overflowing one gives unspecified codes for its block); alpha = RN(1 / (g_x g_R)) in
 * binary64, and the blob holds D(L2^T / alpha) in SVDQ_SEC_L2T. svdq_linear then computes
 * Y = D(alpha * (Q(z_x) Q(z_R) + down (L2^T / alpha)^T) [+ bias]). left_out, right_out,
 * residual_out receive the unscaled factors and R as svdq_prepare's do. fmt is SVDQ_FMT_MX,
 * bits 4. Errors as svdq_prepare, plus EINVAL for x_global_scale outside the range. */
int svdq_prepare_two_level(const void* weight, int64_t M, int64_t N, int64_t ldw, const float* scale,
                           int64_t rank, float x_global_scale, int dtype, void* blob_host,
                           void* left_out, void* right_out, void* residual_out);

/* The same preparation from a weight in the Linear layout ([FI] Parameters: the weight as
 * [n, k], output channels by input channels): weight_nm is [N, M] with host row stride
 * ldw >= M and holds W transposed. The blob (and the optional factor outputs, still in the
 * [M, N] orientation) are byte for byte those of svdq_prepare on W. Errors as svdq_prepare. */
int svdq_prepare_linear(const void* weight_nm, int64_t N, int64_t M, int64_t ldw, const float* scale,
                        int64_t rank, int fmt, int bits, int dtype, void* blob_host,
                        void* left_out, void* right_out, void* residual_out);

/* --------------------------------------------------------------------------------------
 * Workspace of svdq_linear / svdq_quantize_activations: device scratch the caller
 * allocates once (any contents; nothing needs zeroing) and may reuse across calls that are
 * ordered on one stream. Holds activation codes [B, Kp/2] (int8 [B,Kp] for INT bits>4;
 * for MX above 64 rows svdq_linear stores them in 1 KB tiles of 16 rows x 128 codes, rows
 * rounded up to 16), MX scales [B, Kp/32], the down-projection [B, rp], its split-K partials, the
 * per-tensor INT maxima and (svdq_quantize_activations) the reciprocals of the scale.
 * Errors: EINVAL, EDTYPE.
 * ------------------------------------------------------------------------------------ */
int svdq_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t rank, int fmt, int bits, int dtype,
                         size_t* bytes_out);

/* --------------------------------------------------------------------------------------
 * svdq_linear — the per-call hot path ([EX] svdquant_linear, Eq. Y = (X^L1)L2 + Q(X^)Q(R);
 * kernel split after [FI]'s three-step chain). Device call:
 *   (a) X^ = D(x / scale) (binary32 IEEE division), quantised per tensor (INT: s_x from the
 *       global max |X^|) or per 32-block along M (MX), codes packed; fused with
 *   (b) down = X^ L1 (the low-rank branch uses the unquantised X^), fp32 accumulation,
 *       stored in dtype;
 *   (c) Y = D( Q(X^) Q(R) + down L2 ), the residual product on int8 (INT) or block-scaled
 *       FP4 (MX) matrix cores with fp32 (or exact int32) accumulation, the dequant scales
 *       and the up-projection applied in the epilogue.
 *   x: device [B, M] dtype with row stride ldx (unit column stride); blob: device copy of
 *   svdq_prepare's output for the same (M, N, rank, fmt, bits, dtype); y: device [B, N]
 *   dtype with row stride ldy; workspace: >= svdq_workspace_bytes(...).
 * Errors: EINVAL (shape, stride, workspace), EDTYPE, EHIP (launch failure).
 * ------------------------------------------------------------------------------------ */
int svdq_linear(const void* x, int64_t B, int64_t M, int64_t ldx, const void* blob,
                int64_t N, int64_t rank, int fmt, int bits, int dtype,
                void* y, int64_t ldy, void* workspace, size_t workspace_bytes, svdq_stream_t stream);
/* The same with a per-output-channel bias ([FI] Parameters: optional bias of the GEMM):
 * Y = D( Q(X^) Q(R) + down L2 + bias ), bias: device [N] of dtype (or NULL: svdq_linear),
 * added in fp32 before the single output rounding. Errors as svdq_linear, plus EINVAL for
 * a misaligned bias. */
int svdq_linear_bias(const void* x, int64_t B, int64_t M, int64_t ldx, const void* blob,
                     int64_t N, int64_t rank, int fmt, int bits, int dtype, const void* bias,
                     void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                     svdq_stream_t stream);

/* --------------------------------------------------------------------------------------
 * svdq_linear_noalloc — svdq_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The same
 * kernels and results as svdq_linear with no bias (bit for bit), but the workspace is the
 * library's own: a device array of SVDQ_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from
 * the moment the library is loaded on that GPU until the process ends. The call allocates
 * and frees nothing (no hipMalloc/hipFree, no allocating library routine); the caller still
 * passes x, the prepared blob and y. The scratch needs no clearing: every byte a call reads
 * there was written earlier in the same call.
 *   Arguments as svdq_linear without the workspace. `stream` must belong to the current
 *   device (whose scratch the call uses); its address is looked up on the first call on each
 *   device (hipGetSymbolAddress).
 *   Calls on one GPU share its scratch: calls that may overlap in time on one GPU (different
 *   streams, or different host threads without ordering) race and give undefined results;
 *   calls ordered on one stream are safe.
 * Errors: as svdq_linear; EINVAL when the shape's workspace (svdq_workspace_bytes) exceeds
 *   SVDQ_NOALLOC_SCRATCH_BYTES (e.g. MXFP4 bf16 with B * M above ~24 M elements) or the
 *   stream belongs to another device; EUNSUPPORTED for device indices above 63.
 * ------------------------------------------------------------------------------------ */
#define SVDQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int svdq_linear_noalloc(const void* x, int64_t B, int64_t M, int64_t ldx, const void* blob,
                        int64_t N, int64_t rank, int fmt, int bits, int dtype,
                        void* y, int64_t ldy, svdq_stream_t stream);

/* --------------------------------------------------------------------------------------
 * svdq_quantize_activations — step (a) alone, for bit-exact checks ([EX] "Formula and
 * conventions" item 3 for INT; [MS] step 2 for MX). Device call.
 *   x [B,M] dtype row stride ldx; scale [M] f32 device.
 *   codes_out: [B, ldc] bytes; row b holds ceil(M/2) packed 4-bit codes (even m in the low
 *   nibble; INT bits<=4 two's complement, MX E2M1) or M int8 codes for INT bits>4; bytes up
 *   to the padded width Kp/2 (Kp) are written with zero codes, so ldc >= Kp/2 (Kp).
 *   scales_out (MX): [B, lds] E8M0 bytes, ceil(M/32) meaningful per row, lds >= Kp/32.
 *   sx_out (INT): device float* receiving s_x. Unused outputs may be NULL.
 *   workspace: >= svdq_workspace_bytes(B, M, 1, 0, fmt, bits, dtype).
 *   Runs the same kernels as svdq_linear's step (a), with the reciprocals of the scale
 *   (the prepared RECIP section) computed on the device first.
 * ------------------------------------------------------------------------------------ */
int svdq_quantize_activations(const void* x, int64_t B, int64_t M, int64_t ldx, const float* scale,
                              int fmt, int bits, int dtype,
                              void* codes_out, int64_t ldc, void* scales_out, int64_t lds, float* sx_out,
                              void* workspace, size_t workspace_bytes, svdq_stream_t stream);

/* --------------------------------------------------------------------------------------
 * svdq_calibrate_scale — the smoothing scale from a calibration batch (the step before
 * the path): scale_out[m] = max_b |x[b,m]|^alpha / max_n |W[m,n]|^(1-alpha), computed in
 * binary64 and rounded once to float32, and 1 where either maximum is 0. [MS] step 2 names
 * the migration strength iter_smooth.alpha (0.25 in its diffusion example) but prints no
 * formula; this closed form (the SmoothQuant-style balance of the two channel maxima) is the
 * library's reading of it.
 *   x: device [B, M] of dtype, row stride ldx >= M (elements); weight: device [M, N], row
 *   stride ldw >= N; scale_out: device float32 [M] (written); workspace: device, 256-byte
 *   aligned, at least svdq_calibrate_workspace_bytes(B, M) bytes, holding the per-block
 *   column maxima (no zeroing needed). Two kernels on `stream`; asynchronous.
 *   Errors: EDTYPE; EINVAL for NULL buffers, empty shapes, short strides, alpha outside
 *   [0, 1] (or NaN), a small or misaligned workspace, misaligned buffers; EHIP.
 * ------------------------------------------------------------------------------------ */
int svdq_calibrate_workspace_bytes(int64_t B, int64_t M, size_t* bytes_out);
int svdq_calibrate_scale(const void* x, int64_t B, int64_t M, int64_t ldx, const void* weight, int64_t N,
                         int64_t ldw, int dtype, double alpha, float* scale_out, void* workspace,
                         size_t workspace_bytes, svdq_stream_t stream);

/* --------------------------------------------------------------------------------------
 * Kernel timing (profiling aid; not on any page). Between svdq_profile_begin and
 * svdq_profile_end, each svdq_linear call records a HIP event pair around every kernel it
 * launches whose stage bit is set in stage_mask, on the call's stream, for up to max_calls
 * calls (svdq_profile_begin_sampled: only every `every`-th call, counting from the first
 * after the session opens, is recorded, up to max_calls recorded calls). The residual GEMM
 * (stage 3) is a single kernel and its pair is carried by the dispatch itself, so it brackets
 * the kernel's execution; the other stages' pairs bracket their launches on the stream.
 * Stages: 0 = per-tensor max pre-pass (INT), 1 = smooth+quantise+down-projection,
 * 2 = reserved (no kernel; split-K partials of the down-projection are summed in the GEMM
 * epilogue), 3 = residual GEMM + epilogue; a stage that did not run or was not selected
 * reads 0. Each event pair costs host time per call, so a throughput
 * measurement should select only the stages it needs.
 *   svdq_profile_begin: creates the events (host call; no device memory). EINVAL if
 *     max_calls < 1, stage_mask selects no stage or a bit above 3, or a session is already
 *     open; EHIP if event creation fails.
 *   svdq_profile_end: waits for the recorded events, writes ms[call * SVDQ_NSTAGES + stage]
 *     for the n_calls (<= cap) calls recorded, destroys the events and closes the session.
 * Not thread-safe: one session per process at a time.
 * ------------------------------------------------------------------------------------ */
#define SVDQ_NSTAGES 4
int svdq_profile_begin(int max_calls, unsigned stage_mask);
int svdq_profile_begin_sampled(int max_calls, unsigned stage_mask, int every); /* EINVAL if every < 1 */
int svdq_profile_end(float* ms, int cap, int* n_calls);

/* --------------------------------------------------------------------------------------
 * Measured ceilings (measurement aid; not on any page): kernels that run what the operator's
 * kernels are bound by, with nothing else, so that their times can be reported against what
 * the chip sustains as well as against its datasheet peaks.
 *   kind 0: a loop of v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands (unit scales) on
 *     register operands, two waves per SIMD, eight independent accumulators per wave;
 *     arg = loop iterations (>= 1).
 *   kind 1: the same with v_mfma_i32_32x32x32_i8; arg = loop iterations.
 *   kind 2: a grid-stride read of buf[0, buf_bytes) (device, 16-byte aligned, >= 16 bytes) in
 *     16-byte loads by arg 256-thread blocks (1 .. 2^20); buf_bytes rounded down to 16.
 * out: device float32 scratch of out_bytes bytes (kinds 0-1: 8 floats per compute unit;
 * kind 2: 1 KB per block); its contents are unspecified afterwards. work_out (host): flops
 * (kinds 0-1) or bytes (kind 2) of the launch. One kernel on `stream`; asynchronous.
 * Errors: EINVAL for an unknown kind, an argument out of range, NULL or short buffers; EHIP.
 * ------------------------------------------------------------------------------------ */
int svdq_ceiling(int kind, int64_t arg, const void* buf, size_t buf_bytes, float* out, size_t out_bytes,
                 svdq_stream_t stream, double* work_out);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H */
