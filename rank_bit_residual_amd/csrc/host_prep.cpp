// Host side of libsvdq: argument checks, dtype conversion, the one-time weight preparation
// (fold the smoothing scale into W, truncated SVD split, residual, residual quantisation and
// packing into the prepared blob) and the host-only C ABI calls.
//
// Page references (title, section):
//   "SVDQuant Smoothing, Low-rank and Residual Quantization" — "Functions / Return
//     requirements" (_check_smoothing, _check_rank, split_weight) and "Formula and
//     conventions" items 1-3 (ws = scale[:,None] * W; truncated SVD; quantise R, not ws;
//     per-tensor INT with ties to even).
//   "SVDQuant 参数配置流程指南" (msModelSlim), step 2: MXFP4 per_block minmax weights.
//   "flashinfer.gemm.svdquant_linear": invariant per-layer transforms prepared offline,
//     rank a multiple of 32 (we zero-pad instead), residual codes stored per output column
//     with K contiguous.
//
// Built without FP contraction: every quantity that decides a code is one IEEE binary32
// operation, as in the definition.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "host_svd.h"
#include "svdq_internal.h"

namespace svdq {

namespace {
// A fixed buffer rather than a std::string: thread-local storage with no destructor, so
// nothing of the library runs at thread or process exit (after the HIP runtime or a
// profiler attached to it may already have shut down).
constexpr size_t kErrLen = 512;
thread_local char g_last_error[kErrLen];
}  // namespace

int set_error(int status, const std::string& msg) {
  const size_t n = std::min(msg.size(), kErrLen - 1);
  std::memcpy(g_last_error, msg.data(), n);
  g_last_error[n] = '\0';
  return status;
}
void clear_error() { g_last_error[0] = '\0'; }

int check_dtype(int dtype) {
  if (dtype == SVDQ_F32 || dtype == SVDQ_BF16) return SVDQ_OK;
  if (dtype == SVDQ_F64) return set_error(SVDQ_EDTYPE, "float64 is not supported by the device library");
  return set_error(SVDQ_EDTYPE, "unknown dtype code " + std::to_string(dtype));
}

int check_format(int fmt, int bits) {
  if (fmt == SVDQ_FMT_INT) {
    if (bits < 2 || bits > 8) return set_error(SVDQ_EINVAL, "bits must be in [2, 8]");
    return SVDQ_OK;
  }
  if (fmt == SVDQ_FMT_MX) {
    if (bits != 4) return set_error(SVDQ_EINVAL, "MXFP4 uses 4-bit codes (bits must be 4)");
    return SVDQ_OK;
  }
  return set_error(SVDQ_EINVAL, "unknown format code " + std::to_string(fmt));
}

int check_int_accumulation(int64_t M, int fmt, int bits) {
  if (fmt != SVDQ_FMT_INT) return SVDQ_OK;
  const int64_t qmax = ((int64_t)1 << (bits - 1)) - 1;
  const int64_t prod = qmax * qmax * (bits <= 4 ? 256 : 1);
  const int64_t Kp = (M + 255) / 256 * 256;
  if (Kp > (((int64_t)1 << 31) - 1) / prod)
    return set_error(SVDQ_EUNSUPPORTED, "INT residual: M too large for exact int32 accumulation (M rounded up to "
                                        "256, times the largest code product, must stay below 2^31)");
  return SVDQ_OK;
}

void blob_layout(const Dims& d, int64_t off[SVDQ_NSEC]) {
  int64_t o = 0;
  auto sec = [&](int id, int64_t bytes) {
    off[id] = o;
    o = round_up(o + bytes, kAlign);
  };
  sec(SVDQ_SEC_SCALE, d.M * 4);
  sec(SVDQ_SEC_RCODES, d.Np * d.code_row_bytes());
  sec(SVDQ_SEC_RSCALES, d.fmt == SVDQ_FMT_MX ? d.Np * d.mx_scale_row_bytes() : 16);
  sec(SVDQ_SEC_L1T, d.rp * d.Kp * (int64_t)dtype_size(d.dtype));
  sec(SVDQ_SEC_L2T, d.Np * d.rp * (int64_t)dtype_size(d.dtype));
  sec(SVDQ_SEC_RECIP, d.M * 4);
  sec(SVDQ_SEC_GLOBAL, 16);
  off[SVDQ_SEC_END] = o;
}

namespace {

// ---- dtype conversion (finite values) --------------------------------------------------
inline float bf16_bits_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint16_t float_to_bf16_bits(float f) {  // round to nearest, ties to even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// double -> bf16 with a single rounding: scale by the spacing of bf16 numbers around v.
inline uint16_t double_to_bf16_bits(double v) {
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0;
  const int e = std::max(std::ilogb(v), -126);
  const double q = std::ldexp(1.0, e - 7);
  const float r = (float)(std::nearbyint(v / q) * q);  // exact: <= 8 significant bits
  uint32_t u;
  std::memcpy(&u, &r, 4);
  return (uint16_t)(u >> 16);
}

struct HostMat {  // read-only view of a dtype matrix on the host: element (i, j)
  const void* p;
  int64_t ld;
  int dtype;
  bool trans = false;  // stored transposed: (i, j) at p[j * ld + i]
  float at(int64_t i, int64_t j) const {
    const int64_t k = trans ? j * ld + i : i * ld + j;
    if (dtype == SVDQ_F32) return ((const float*)p)[k];
    return bf16_bits_to_float(((const uint16_t*)p)[k]);
  }
};

// Store a float that is already representable in dtype.
inline void store_exact(void* base, int64_t idx, int dtype, float v) {
  if (dtype == SVDQ_F32)
    ((float*)base)[idx] = v;
  else
    ((uint16_t*)base)[idx] = float_to_bf16_bits(v);
}
// Round a binary32 result to dtype (RNE for bf16).
inline float round_f32(float v, int dtype) { return dtype == SVDQ_F32 ? v : bf16_bits_to_float(float_to_bf16_bits(v)); }
// Round a float64 result to dtype with one rounding.
inline float round_f64(double v, int dtype) {
  return dtype == SVDQ_F32 ? (float)v : bf16_bits_to_float(double_to_bf16_bits(v));
}

// ---- quantisers ------------------------------------------------------------------------
// MXFP4 shared exponent: smallest e with a <= 6 * 2^e (clamped to [-127, 127]).
// For normal a = 1.m * 2^E: e = E - 2 when 1.m <= 1.5, else E - 1; a < 2^-126 gives -127.
inline int mx_exponent(float a) {
  uint32_t u;
  std::memcpy(&u, &a, 4);
  const int be = (int)((u >> 23) & 0xFF);
  const uint32_t mant = u & 0x7FFFFFu;
  if (be == 0) return -127;
  const int e = (be - 127) - 2 + (mant > 0x400000u ? 1 : 0);
  return std::min(127, std::max(-127, e));
}
// E2M1 code of z / 2^e: magnitude thresholds are the midpoints of {0,.5,1,1.5,2,3,4,6};
// at a midpoint the even code wins (0.25->0, 0.75->2, 1.25->2, 1.75->4, 2.5->4, 3.5->6, 5->6).
inline uint8_t e2m1_code(float z, int e) {
  const float v = std::ldexp(std::fabs(z), -e);
  const int c = (v > 0.25f) + (v >= 0.75f) + (v > 1.25f) + (v >= 1.75f) + (v > 2.5f) + (v >= 3.5f) + (v > 5.0f);
  return (uint8_t)(c | (std::signbit(z) ? 8 : 0));
}

// Stage-tiled E8M0 index (the device kernels' layout): for each 64-row group and each
// 128-code K stage, the 64 rows' four block bytes are contiguous.
inline int64_t mx_tiled(int64_t row, int64_t kb, int64_t kq) {
  return (((row >> 6) * kq + (kb >> 2)) << 8) + ((row & 63) << 2) + (kb & 3);
}

// Tiled MXFP4 residual codes: byte j (codes 2j, 2j+1) of column n sits at
// ((n/16) * kq + j/64) * 1024 + (n%16) * 64 + j%64, i.e. every 16-column x 128-code block
// is 1 KB contiguous, the operand of one wave-wide load.
inline int64_t mx_code_tiled(int64_t n, int64_t j, int64_t kq) {
  return (((n >> 4) * kq + (j >> 6)) << 10) + ((n & 15) << 6) + (j & 63);
}

int validate_prepare(int64_t M, int64_t N, int64_t ldw, int64_t rank, int fmt, int bits, int dtype) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_format(fmt, bits))) return st;
  if (M < 1 || N < 1) return set_error(SVDQ_EINVAL, "weight must be a nonempty matrix");
  if (ldw < N) return set_error(SVDQ_EINVAL, "weight row stride smaller than N");
  if (rank < 0 || rank > std::min(M, N)) return set_error(SVDQ_EINVAL, "rank must be in [0, min(M, N)]");
  return check_int_accumulation(M, fmt, bits);
}

// Split ws [M,N] (float values exact in dtype) into rounded factors and the residual.
// Where the truncated SVD runs: the host, or the GPU for the randomized route's products.
struct SplitDevice {
  void* workspace = nullptr;
  void* stream = nullptr;
  int hip_error = 0;
};

void split(const std::vector<float>& ws, int64_t M, int64_t N, int64_t rank, int dtype, std::vector<float>& L1,
           std::vector<float>& L2, std::vector<float>& R, SplitDevice* dev = nullptr) {
  L1.assign((size_t)(M * rank), 0.f);
  L2.assign((size_t)(rank * N), 0.f);
  R.assign((size_t)(M * N), 0.f);
  if (rank == 0) {
    R = ws;
    return;
  }
  std::vector<double> l1((size_t)(M * rank)), l2((size_t)(rank * N));
  if (dev)
    dev->hip_error = run_split_on_device(ws.data(), M, N, rank, dev->workspace, dev->stream, l1.data(), l2.data());
  else
    host::truncated_svd(ws.data(), M, N, N, rank, l1.data(), l2.data());
  for (size_t i = 0; i < l1.size(); i++) L1[i] = round_f64(l1[i], dtype);
  for (size_t i = 0; i < l2.size(); i++) L2[i] = round_f64(l2[i], dtype);
  // R = D(ws - L1 L2), the product in float64 from the stored factors
  std::vector<double> prod((size_t)(M * N));
  host::gemm<float, float>(M, N, rank, L1.data(), rank, 1, L2.data(), N, 1, prod.data(), N);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M * N; i++) R[i] = round_f64((double)ws[i] - prod[i], dtype);
}

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" {

const char* svdq_last_error(void) { return g_last_error; }

const char* svdq_version(void) { return "svdq 0.1 gfx950"; }

int svdq_check_smoothing(int64_t B, int64_t M, int64_t Mw, int64_t Ms, int64_t N, const float* scale_host) {
  clear_error();
  if (B < 1 || M < 1 || N < 1 || Mw < 1 || Ms < 1) return set_error(SVDQ_EINVAL, "x, weight and scale must be nonempty");
  if (M != Mw || M != Ms) return set_error(SVDQ_EINVAL, "input-channel sizes of x, weight and scale differ");
  if (!scale_host) return set_error(SVDQ_EINVAL, "scale is NULL");
  for (int64_t m = 0; m < M; m++) {
    const float s = scale_host[m];
    if (!(std::isfinite(s) && s > 0.f))
      return set_error(SVDQ_EINVAL, "scale must be positive and finite (index " + std::to_string(m) + ")");
  }
  return SVDQ_OK;
}

int svdq_check_rank(int64_t M, int64_t N, int64_t rank) {
  clear_error();
  if (M < 1 || N < 1) return set_error(SVDQ_EINVAL, "weight must be a nonempty matrix");
  if (rank < 0 || rank > std::min(M, N)) return set_error(SVDQ_EINVAL, "rank must be in [0, min(M, N)]");
  return SVDQ_OK;
}

int svdq_split_weight(const void* weight, int64_t M, int64_t N, int64_t ldw, int dtype, int64_t rank, void* left,
                      void* right, void* residual) {
  clear_error();
  int st = validate_prepare(M, N, ldw, rank, SVDQ_FMT_INT, 4, dtype);
  if (st) return st;
  if (!weight || !residual || (rank > 0 && (!left || !right)))
    return set_error(SVDQ_EINVAL, "NULL buffer passed to split_weight");
  HostMat W{weight, ldw, dtype};
  std::vector<float> ws((size_t)(M * N));
  for (int64_t i = 0; i < M; i++)
    for (int64_t j = 0; j < N; j++) ws[i * N + j] = W.at(i, j);
  std::vector<float> L1, L2, R;
  split(ws, M, N, rank, dtype, L1, L2, R);
  for (int64_t i = 0; i < M * rank; i++) store_exact(left, i, dtype, L1[i]);
  for (int64_t i = 0; i < rank * N; i++) store_exact(right, i, dtype, L2[i]);
  for (int64_t i = 0; i < M * N; i++) store_exact(residual, i, dtype, R[i]);
  return SVDQ_OK;
}

int svdq_prepared_layout(int64_t M, int64_t N, int64_t rank, int fmt, int bits, int dtype, int64_t offsets[SVDQ_NSEC]) {
  clear_error();
  int st = validate_prepare(M, N, N, rank, fmt, bits, dtype);
  if (st) return st;
  blob_layout(make_dims(M, N, rank, fmt, bits, dtype), offsets);
  return SVDQ_OK;
}

static int prepare_impl(const HostMat& W, int64_t M, int64_t N, const float* scale, int64_t rank, int fmt, int bits,
                        int dtype, void* blob_host, void* left_out, void* right_out, void* residual_out,
                        SplitDevice* dev = nullptr, float x_gscale = 0.f);

int svdq_prepare_gpu_workspace_bytes(int64_t M, int64_t N, int64_t rank, size_t* bytes_out) {
  clear_error();
  if (!bytes_out) return set_error(SVDQ_EINVAL, "bytes_out is NULL");
  if (M < 1 || N < 1 || rank < 0 || rank > std::min(M, N)) return set_error(SVDQ_EINVAL, "bad shape or rank");
  const int64_t k = device_svd_columns(M, N, rank);
  *bytes_out = k ? device_svd_bytes(M, N, k, rank) : 0;
  return SVDQ_OK;
}

int svdq_prepare_gpu(const void* weight, int64_t M, int64_t N, int64_t ldw, const float* scale, int64_t rank, int fmt,
                     int bits, int dtype, void* blob_host, void* left_out, void* right_out, void* residual_out,
                     void* workspace, size_t workspace_bytes, svdq_stream_t stream) {
  clear_error();
  int st = validate_prepare(M, N, ldw, rank, fmt, bits, dtype);
  if (st) return st;
  if (!weight || !scale || !blob_host) return set_error(SVDQ_EINVAL, "NULL buffer passed to prepare");
  size_t need = 0;
  if ((st = svdq_prepare_gpu_workspace_bytes(M, N, rank, &need))) return st;
  if (need && (!workspace || workspace_bytes < need || (uintptr_t)workspace % kAlign))
    return set_error(SVDQ_EINVAL, "device workspace too small or not 256-byte aligned");
  SplitDevice dev{workspace, (void*)stream, 0};
  st = prepare_impl(HostMat{weight, ldw, dtype, false}, M, N, scale, rank, fmt, bits, dtype, blob_host, left_out,
                    right_out, residual_out, &dev);
  if (st) return st;
  if (dev.hip_error) return set_error(SVDQ_EHIP, "truncated SVD on the device failed");
  return SVDQ_OK;
}

int svdq_prepare(const void* weight, int64_t M, int64_t N, int64_t ldw, const float* scale, int64_t rank, int fmt,
                 int bits, int dtype, void* blob_host, void* left_out, void* right_out, void* residual_out) {
  clear_error();
  int st = validate_prepare(M, N, ldw, rank, fmt, bits, dtype);
  if (st) return st;
  if (!weight || !scale || !blob_host) return set_error(SVDQ_EINVAL, "NULL buffer passed to prepare");
  return prepare_impl(HostMat{weight, ldw, dtype, false}, M, N, scale, rank, fmt, bits, dtype, blob_host, left_out,
                      right_out, residual_out);
}

int svdq_prepare_two_level(const void* weight, int64_t M, int64_t N, int64_t ldw, const float* scale, int64_t rank,
                           float x_global_scale, int dtype, void* blob_host, void* left_out, void* right_out,
                           void* residual_out) {
  clear_error();
  int st = validate_prepare(M, N, ldw, rank, SVDQ_FMT_MX, 4, dtype);
  if (st) return st;
  if (!weight || !scale || !blob_host) return set_error(SVDQ_EINVAL, "NULL buffer passed to prepare");
  if (!(x_global_scale >= 0x1p-64f && x_global_scale <= 0x1p64f))
    return set_error(SVDQ_EINVAL, "x_global_scale must be finite and in [2^-64, 2^64]");
  return prepare_impl(HostMat{weight, ldw, dtype, false}, M, N, scale, rank, SVDQ_FMT_MX, 4, dtype, blob_host,
                      left_out, right_out, residual_out, nullptr, x_global_scale);
}

int svdq_prepare_linear(const void* weight_nm, int64_t N, int64_t M, int64_t ldw, const float* scale, int64_t rank,
                        int fmt, int bits, int dtype, void* blob_host, void* left_out, void* right_out,
                        void* residual_out) {
  clear_error();
  // validate as the [M, N] matrix it is the transpose of; the row stride runs over M here
  int st = validate_prepare(M, N, N, rank, fmt, bits, dtype);
  if (st) return st;
  if (ldw < M) return set_error(SVDQ_EINVAL, "weight row stride smaller than M");
  if (!weight_nm || !scale || !blob_host) return set_error(SVDQ_EINVAL, "NULL buffer passed to prepare");
  return prepare_impl(HostMat{weight_nm, ldw, dtype, true}, M, N, scale, rank, fmt, bits, dtype, blob_host, left_out,
                      right_out, residual_out);
}

// x_gscale > 0: MX two-level scaling with that activation global scale (see
// svdq_prepare_two_level); 0: plain preparation (SVDQ_SEC_GLOBAL = {1, 1, 1, 0}).
static int prepare_impl(const HostMat& W, int64_t M, int64_t N, const float* scale, int64_t rank, int fmt, int bits,
                        int dtype, void* blob_host, void* left_out, void* right_out, void* residual_out,
                        SplitDevice* dev, float x_gscale) {
  int st;
  if ((st = svdq_check_smoothing(1, M, M, M, N, scale))) return st;
  const Dims d = make_dims(M, N, rank, fmt, bits, dtype);
  int64_t off[SVDQ_NSEC];
  blob_layout(d, off);
  uint8_t* blob = (uint8_t*)blob_host;
  std::memset(blob, 0, (size_t)off[SVDQ_SEC_END]);

  // fold: ws = D(scale[m] * W[m,n]), one binary32 multiply and one rounding
  std::vector<float> ws((size_t)(M * N));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; i++)
    for (int64_t j = 0; j < N; j++) ws[i * N + j] = round_f32(scale[i] * W.at(i, j), dtype);

  std::vector<float> L1, L2, R;
  split(ws, M, N, rank, dtype, L1, L2, R, dev);

  std::memcpy(blob + off[SVDQ_SEC_SCALE], scale, (size_t)M * 4);
  {
    // correctly rounded reciprocals for the device's fast exact division (0 = use IEEE division)
    float* rc = reinterpret_cast<float*>(blob + off[SVDQ_SEC_RECIP]);
    for (int64_t m = 0; m < M; m++) {
      const float sv = scale[m];
      rc[m] = (sv >= 0x1p-90f && sv <= 0x1p90f) ? 1.0f / sv : 0.0f;
    }
  }

  // two-level scaling (MX): the residual's global scale g_R maps max|R| onto 6 * 2^ex (see
  // svdq_prepare_two_level), alpha = RN(1 / (g_x g_R)) in binary64
  float g_resid = 1.f, alpha = 1.f;
  if (x_gscale > 0.f) {
    float a = 0.f;
    for (float v : R) a = std::max(a, std::fabs(v));
    if (a > 0.f) {
      int ex = 0;
      (void)std::frexp((double)a / 6.0, &ex);
      g_resid = (float)(std::ldexp(6.0, ex) / (double)a);
    }
    alpha = (float)(1.0 / ((double)x_gscale * (double)g_resid));
  }
  {
    const float gl[4] = {x_gscale > 0.f ? x_gscale : 1.f, g_resid, alpha, 0.f};
    std::memcpy(blob + off[SVDQ_SEC_GLOBAL], gl, sizeof gl);
  }

  uint8_t* codes = blob + off[SVDQ_SEC_RCODES];
  const int64_t crow = d.code_row_bytes();
  if (fmt == SVDQ_FMT_INT) {
    // one scale for the whole residual: s = max|R| / qmax, codes = clamp(rint(R / s))
    const int qmax = (1 << (bits - 1)) - 1;
    float a = 0.f;
    for (float v : R) a = std::max(a, std::fabs(v));
    const float s = a / (float)qmax;
    std::memcpy(blob + off[SVDQ_SEC_RSCALES], &s, 4);
    if (a > 0.f) {
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < N; n++) {
        for (int64_t m = 0; m < M; m++) {
          const float q = R[m * N + n] / s;
          const int c = (int)std::max<float>(-(float)qmax, std::min<float>((float)qmax, std::nearbyint(q)));
          if (d.nibbles())
            codes[n * crow + m / 2] |= (uint8_t)((c & 0xF) << (4 * (m & 1)));
          else
            codes[n * crow + m] = (uint8_t)(int8_t)c;
        }
      }
    }
  } else {
    // MXFP4 per column n of z = RN(R * g_R) (g_R = 1 without two-level scaling), 32-element
    // blocks along m
    const float gr = g_resid;
    uint8_t* sc = blob + off[SVDQ_SEC_RSCALES];
    const int64_t nb = ceil_div(M, kMxBlock);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
      for (int64_t b = 0; b < nb; b++) {
        const int64_t m0 = b * kMxBlock, m1 = std::min(M, m0 + kMxBlock);
        float a = 0.f;
        for (int64_t m = m0; m < m1; m++) a = std::max(a, std::fabs(R[m * N + n] * gr));
        const int e = mx_exponent(a);
        sc[mx_tiled(n, b, d.Kp / 128)] = (uint8_t)(e + 127);
        for (int64_t m = m0; m < m1; m++)
          codes[mx_code_tiled(n, m / 2, d.Kp / 128)] |= (uint8_t)(e2m1_code(R[m * N + n] * gr, e) << (4 * (m & 1)));
      }
    }
  }
  // low-rank factors, transposed and zero-padded: L1^T [rp, Kp] in 16x128 matrix-core tiles,
  // L2^T [Np, rp] row-major
  void* l1t = blob + off[SVDQ_SEC_L1T];
  void* l2t = blob + off[SVDQ_SEC_L2T];
  const int64_t E = 16 / dtype_size(dtype);
  for (int64_t t = 0; t < rank; t++)
    for (int64_t m = 0; m < M; m++) {
      const int64_t tile = (t / 16) * (d.Kp / 128) + m / 128;
      const int64_t in_tile = ((((m % 32) / E) * 4 + (m % 128) / 32) * 16 + t % 16) * E + m % E;
      store_exact(l1t, tile * 2048 + in_tile, dtype, L1[m * rank + t]);
    }
  // (two-level: the up-projection factor divided by alpha, rounded to the dtype)
  for (int64_t n = 0; n < N; n++)
    for (int64_t t = 0; t < rank; t++) {
      const float v = alpha == 1.f ? L2[t * N + n] : round_f64((double)L2[t * N + n] / (double)alpha, dtype);
      store_exact(l2t, n * d.rp + t, dtype, v);
    }

  if (left_out)
    for (int64_t i = 0; i < M * rank; i++) store_exact(left_out, i, dtype, L1[i]);
  if (right_out)
    for (int64_t i = 0; i < rank * N; i++) store_exact(right_out, i, dtype, L2[i]);
  if (residual_out)
    for (int64_t i = 0; i < M * N; i++) store_exact(residual_out, i, dtype, R[i]);
  return SVDQ_OK;
}

}  // extern "C"
