// Internal helpers shared by the host preparation code and the device launch code of
// libsvdq: status/error plumbing, padded sizes and the prepared-blob / workspace layouts.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/svdq.h"

namespace svdq {

constexpr int64_t kKPad = 256;   // K (= M) padding: one 128-byte LDS stage of packed 4-bit codes
constexpr int64_t kNPad = 256;   // N padding of the prepared weight: the widest GEMM tile
constexpr int64_t kRPad = 32;    // rank padding: the bf16 MFMA K-step of the low-rank GEMMs
constexpr int64_t kAlign = 256;  // byte alignment of every blob / workspace section
constexpr int kMxBlock = 32;     // MXFP4 block length along K

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }

// Thread-local last-error message; set_error returns the status for `return set_error(...)`.
int set_error(int status, const std::string& msg);
void clear_error();

inline size_t dtype_size(int dtype) { return dtype == SVDQ_F32 ? 4 : 2; }

// Validates (dtype, fmt, bits) and returns SVDQ_OK or the error status (message set).
int check_dtype(int dtype);
int check_format(int fmt, int bits);
// INT residual products accumulate exactly in int32 on the matrix cores: Kp (M rounded up to
// 256) times the largest code product (qmax^2, times 256 for 4-bit codes, which the int8
// MFMAs see as 16 c) must stay below 2^31. EUNSUPPORTED otherwise (MX accumulates in fp32).
int check_int_accumulation(int64_t M, int fmt, int bits);

struct Dims {
  int64_t M, N, rank;
  int fmt, bits, dtype;
  int64_t Kp, Np, rp;
  bool nibbles() const { return fmt == SVDQ_FMT_MX || bits <= 4; }
  int64_t code_row_bytes() const { return nibbles() ? Kp / 2 : Kp; }  // packed code bytes per row
  int64_t mx_scale_row_bytes() const { return Kp / kMxBlock; }
};

inline Dims make_dims(int64_t M, int64_t N, int64_t rank, int fmt, int bits, int dtype) {
  Dims d{M, N, rank, fmt, bits, dtype, round_up(M, kKPad), round_up(N, kNPad), round_up(rank, kRPad)};
  return d;
}

// Byte offsets of the prepared-blob sections (see svdq.h).
void blob_layout(const Dims& d, int64_t off[SVDQ_NSEC]);

// Workspace sections of svdq_linear.
enum { WS_CODES = 0, WS_SCALES, WS_DOWN, WS_PARTIAL, WS_AMAX, WS_SX, WS_RECIP, WS_END, WS_NSEC };
struct LaunchPlan {
  int64_t B;
  int row_blocks;   // activation row blocks of kernel (a) (16 rows each)
  int rchunk;       // low-rank columns per block of kernel (a): 32 (rank <= 32) or 64, 16 for small batches
  int r_chunks;     // rchunk-wide low-rank column chunks of kernel (a)
  int k_chunks;     // split of K in kernel (a) (down-projection partials when > 1)
  int k_chunk_len;  // K columns per chunk (multiple of 128)
  int amax_cols, amax_rows;  // grid of the INT per-tensor max pre-pass
  int amax_blocks;           // amax_cols * amax_rows partial maxima
};
LaunchPlan make_plan(const Dims& d, int64_t B);

// Truncated SVD on the GPU (k_svd.hip): the randomized route's subspace iteration and
// Rayleigh-Ritz step in float64 on the device, for A [M x N] float32 row-major on the host.
// device_svd_columns: the panel width k of that route (0: the host takes the whole split —
// the full Jacobi route of small matrices, or panels wider than the device route's kMaxDeviceK);
// workspace: device, >= device_svd_bytes(M, N, k, r); stream: a hipStream_t. Returns the first
// HIP error (0 = none).
constexpr int64_t kMaxDeviceK = 256;
int64_t device_svd_columns(int64_t M, int64_t N, int64_t r);
size_t device_svd_bytes(int64_t M, int64_t N, int64_t k, int64_t r);
int run_split_on_device(const float* A, int64_t M, int64_t N, int64_t r, void* workspace, void* stream, double* L1,
                        double* L2);
void workspace_layout(const Dims& d, const LaunchPlan& p, int64_t off[WS_NSEC]);

}  // namespace svdq
