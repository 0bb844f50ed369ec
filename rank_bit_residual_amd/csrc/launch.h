// Kernel launchers of libsvdq (device code in k_act.hip / k_gemm.hip, called from capi.hip).
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

struct ActParams {
  const void* x;
  int64_t ldx;
  int B, M, Kp;
  const float* scale;
  const float* recip;  // RN(1/scale), 0 where the scale lies outside [2^-90, 2^90]
  uint8_t* codes;  // [B][ldc] bytes, or NULL (down-projection only)
  int64_t ldc;
  uint8_t* mxs;  // MX scales: row-major [B][lds], or stage-tiled when mxs_tiled
  int64_t lds;
  int mxs_tiled;
  // MX: codes in 1 KB tiles of 16 rows x 128 codes (tile (b / 16, k / 128) at
  // ((b / 16) * Kp / 128 + k / 128) * 1024, row b % 16 at 64 (b % 16)) instead of row-major,
  // for the large-batch MXFP4 GEMM; rows up to the next multiple of 16 must be allocated
  int codes_tiled;
  const float* amax_part;  // INT: per-block maxima of |X^|
  int n_amax;
  int bits;
  float* sx_out;  // INT: receives s_x (may be NULL)
  const void* l1t;  // [rp][Kp] dtype
  int rp;
  float* down_part;  // [k_chunks][rp / 16][B][16] f32 when k_chunks > 1 (part_index)
  void* down;        // [B][rp] dtype when k_chunks == 1
  int k_chunks, k_chunk_len;
  int x_vec_ok;  // x base and row stride allow 16-byte loads
  const float* gscale;  // MX: the activation global scale g_x (codes of RN(X^ g_x)), or NULL
};

struct GemmParams {
  const uint8_t* acodes;  // row-major [B][lda], or (MX, acodes_tiled) 16-row x 128-code tiles
  int64_t lda;
  int acodes_tiled;
  const uint8_t* ascales;  // stage-tiled E8M0 bytes (see mx_scale_tiled_index)
  int ascale_groups;       // 64-row groups of the activation scales
  const uint8_t* wcodes;
  int64_t ldw;
  const uint8_t* wscales;  // stage-tiled E8M0 bytes over npad rows
  int kq;                  // Kp / 128: 128-code stages per row
  const float* sx;
  const float* sr;
  const void* down;         // [B][rp] dtype, when down_chunks == 1
  const float* down_part;   // [down_chunks][rp / 16][B][16] f32 split-K partials of X^ L1 (part_index), when down_chunks > 1
  int down_chunks;
  const void* l2t;
  int rp;
  void* y;
  int64_t ldy;
  const void* bias;  // [N] dtype added before the output rounding, or nullptr
  const float* alpha;  // MX: residual-plus-up-projection scale applied before the bias, or nullptr
  int B, N, kstages;
  int npad;  // rows of the prepared weight (N rounded up); loads clamp to npad - 1
};

hipError_t launch_smooth(const void* x, int64_t B, int64_t M, int64_t sxb, int64_t sxm, const void* w, int64_t N,
                         int64_t swm, int64_t swn, const float* scale, int dtype, void* xs, int64_t ldxs, void* ws,
                         int64_t ldws, hipStream_t stream);
// Per-block maxima of |D(x / scale)| for the per-tensor INT scale, col_blocks = ceil(M / 2048)
// by row_blocks blocks, into part[col_blocks * row_blocks].
hipError_t launch_amax_smoothed(const void* x, int B, int M, int64_t ldx, const float* scale, const float* recip,
                                int dtype, float* part, int col_blocks, int row_blocks, hipStream_t stream);
// Per-block maxima of |z| (smoothed by `scale` when non-NULL) into part[nparts].
hipError_t launch_amax(const void* z, int64_t rows, int64_t cols, int64_t szr, int64_t szc, const float* scale,
                       int dtype, float* part, int nparts, hipStream_t stream);
hipError_t launch_fake_quant(const void* z, int64_t rows, int64_t cols, int64_t szr, int64_t szc, int dtype, int bits,
                             const float* part, int nparts, void* out, int64_t ldo, float* s_out, hipStream_t stream);
// recip[m] = RN(1 / scale[m]) for scale[m] in [2^-90, 2^90], else 0 (the prepared RECIP section).
hipError_t launch_reciprocals(const float* scale, int M, float* recip, hipStream_t stream);
// grid (row_blocks, p.k_chunks, r_chunks) of blocks covering rchunk (16, 32 or 64) low-rank columns each
hipError_t launch_act_quant(const ActParams& p, int fmt, int dtype, int row_blocks, int r_chunks, int rchunk,
                            hipStream_t stream);

// Kernel-timing events for the residual GEMM launch of the current call (svdq_profile_begin):
// when set, the GEMM launchers pass them to the dispatch itself (hipExtLaunchKernelGGL), so
// they bracket the kernel's execution and not the queue gap before it.
struct GemmEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local GemmEvents g_gemm_events;

template <class K, class... Args>
inline hipError_t launch_gemm_kernel(K kernel, dim3 grid, dim3 block, unsigned shmem, hipStream_t stream, Args... args) {
  if (g_gemm_events.start)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, g_gemm_events.start, g_gemm_events.stop, 0u, args...);
  else
    kernel<<<grid, block, shmem, stream>>>(args...);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, int fmt, int bits, int dtype, hipStream_t stream);
// Smoothing-scale calibration: per-column maxima of |x| into part[calib_parts(B, M)][M], then
// scale[m] from them and the row maxima of |W|.
int calib_parts(int64_t B, int64_t M);
hipError_t launch_calibrate(const void* x, int B, int M, int64_t ldx, const void* w, int N, int64_t ldw, int dtype,
                            double alpha, float* part, float* scale, hipStream_t stream);
// Large-batch MXFP4 kernel; hipErrorNotSupported (nothing launched) when the shape is not covered
// (mx_large_accepts false) or the activation codes are not tiled.
hipError_t launch_gemm_mx_large(const GemmParams& p, int dtype, hipStream_t stream);
// Whether launch_gemm_mx_large takes this shape (p.kstages in 64-byte stages); the caller then
// has the activation kernel write tiled codes.
bool mx_large_accepts(const GemmParams& p);
// Per-tensor INT: 64x64 tiles, K split over the waves of a block (kstages = Kp/256 for nibble
// codes, Kp/128 for int8 codes; any K).
hipError_t launch_gemm_int4(const GemmParams& p, int bits, int dtype, hipStream_t stream);
// Per-tensor INT (nibble or int8 codes) on the large-batch tiles; hipErrorNotSupported (nothing
// launched) when the shape is better served by launch_gemm_int4.
hipError_t launch_gemm_int_big(const GemmParams& p, int bits, int dtype, hipStream_t stream);
// MXFP4, B <= 64 (bf16 or f32 io): K split over waves, weights streamed straight into registers.
hipError_t launch_gemm_mx_decode(const GemmParams& p, int dtype, hipStream_t stream);

// Ceiling probes (k_ceiling.hip): kind 0 FP4 MFMA loop, 1 INT8 MFMA loop (arg = iterations),
// 2 read stream over buf[0, bytes) (arg = 256-thread blocks); *work = flops or bytes of one launch.
hipError_t launch_ceiling(int kind, int64_t arg, const void* buf, size_t bytes, float* out, size_t out_bytes,
                          hipStream_t stream, double* work);

}  // namespace svdq
