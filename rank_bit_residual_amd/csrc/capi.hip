// Device-side C ABI of libsvdq: argument validation, launch plans, workspace layout and the
// launch sequences of svdq_linear (steps a+b, then c, whose epilogue sums split-K partials),
// svdq_quantize_activations, svdq_fake_quantize and svdq_smooth_inputs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <string>
#include <type_traits>

#include "launch.h"
#include "svdq_internal.h"

namespace svdq {

LaunchPlan make_plan(const Dims& d, int64_t B) {
  LaunchPlan p;
  p.B = B;
  p.row_blocks = (int)ceil_div(B, 16);
  // 16-wide rank chunks when 64-wide ones would leave most of the chip idle (decode batches);
  // otherwise one 32-wide chunk for ranks up to 32 (its operands travel a step ahead), else 64
  p.rchunk = (d.rp > 0 && (int64_t)p.row_blocks * ceil_div(d.rp, 64) < 256) ? 16 : (d.rp <= 32 ? 32 : 64);
  p.r_chunks = d.rp > 0 ? (int)ceil_div(d.rp, p.rchunk) : 1;
  // Split K across blocks only when rows x low-rank chunks give fewer than ~256 blocks, and
  // never below one 128-wide step per wave of a block (8 waves: 1024 K per chunk).
  const int64_t per = (int64_t)p.row_blocks * p.r_chunks;
  int64_t chunks = per >= 256 ? 1 : ceil_div(256, per);
  chunks = std::min<int64_t>(chunks, std::max<int64_t>(1, ceil_div(d.Kp, 1024)));
  p.k_chunk_len = (int)round_up(ceil_div(d.Kp, chunks), 128);
  p.k_chunks = (int)ceil_div(d.Kp, p.k_chunk_len);
  p.amax_cols = (int)ceil_div(d.M, 2048);
  // 8 rows per block, fewer (down to 1) while that leaves under 256 blocks, more when that
  // would give over 4096 partial maxima (every wave of the activation kernel reduces them all)
  int64_t amax_rpb = std::max<int64_t>(1, std::min<int64_t>(8, B * p.amax_cols / 256));
  amax_rpb = std::max<int64_t>(amax_rpb, ceil_div(B * p.amax_cols, 4096));
  p.amax_rows = (int)std::min<int64_t>(65535, std::max<int64_t>(1, ceil_div(B, amax_rpb)));
  p.amax_blocks = p.amax_cols * p.amax_rows;
  return p;
}

void workspace_layout(const Dims& d, const LaunchPlan& p, int64_t off[WS_NSEC]) {
  int64_t o = 0;
  auto sec = [&](int id, int64_t bytes) {
    off[id] = o;
    o = round_up(o + bytes, kAlign);
  };
  const int64_t B = p.B;
  sec(WS_CODES, round_up(B, 16) * d.code_row_bytes());  // tiled MX codes fill whole 16-row tiles
  sec(WS_SCALES, d.fmt == SVDQ_FMT_MX ? round_up(B, 64) * d.mx_scale_row_bytes() : 0);  // stage-tiled
  sec(WS_DOWN, B * d.rp * (int64_t)dtype_size(d.dtype));
  sec(WS_PARTIAL, p.k_chunks > 1 ? (int64_t)p.k_chunks * B * d.rp * 4 : 0);
  sec(WS_AMAX, d.fmt == SVDQ_FMT_INT ? (int64_t)p.amax_blocks * 4 : 0);
  sec(WS_SX, 16);
  sec(WS_RECIP, d.Kp * 4);  // svdq_quantize_activations: RN(1/scale) computed on the device
  off[WS_END] = o;
}

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// Kernel-timing session (svdq_profile_begin / svdq_profile_end). Plain data with no
// destructor: the arrays are released by svdq_profile_end, so nothing of this state runs at
// process exit, when the HIP runtime (or a profiler attached to it) may already be gone.
struct Profile {
  bool open;
  int max_calls, calls;  // recorded calls: capacity and count
  int every, seen;       // record calls seen % every == 0
  unsigned mask;         // stages that record events
  hipEvent_t* ev;        // [call][stage][begin, end], max_calls * SVDQ_NSTAGES * 2 (new[])
  uint8_t* recorded;     // [call][stage]: both events of the pair were recorded (new[])
};
Profile g_prof;  // zero-initialised: no session open
static_assert(std::is_trivially_destructible<Profile>::value, "no exit-time destructor");
}  // namespace

thread_local GemmEvents g_gemm_events;

namespace {

struct StageTimer {
  hipStream_t s;
  int call = -1;
  explicit StageTimer(hipStream_t s_) : s(s_) {
    if (g_prof.open && g_prof.calls < g_prof.max_calls && g_prof.seen++ % g_prof.every == 0) call = g_prof.calls++;
  }
  hipEvent_t ev(int stage, int which) const { return g_prof.ev[((size_t)call * SVDQ_NSTAGES + stage) * 2 + which]; }
  bool on(int stage) const { return call >= 0 && ((g_prof.mask >> stage) & 1u); }
  void begin(int stage) const {
    if (on(stage)) hipEventRecord(ev(stage, 0), s);
  }
  void end(int stage) const {
    if (on(stage) && hipEventRecord(ev(stage, 1), s) == hipSuccess)
      g_prof.recorded[(size_t)call * SVDQ_NSTAGES + stage] = 1;
  }
  // The GEMM stage is one kernel: its events ride on the dispatch (g_gemm_events) instead.
  void gemm_begin() const {
    if (on(3)) g_gemm_events = GemmEvents{ev(3, 0), ev(3, 1)};
  }
  void gemm_end(hipError_t launched) const {
    if (on(3) && launched == hipSuccess) g_prof.recorded[(size_t)call * SVDQ_NSTAGES + 3] = 1;
    g_gemm_events = GemmEvents{};
  }
};

// Clears an error left by an earlier, unrelated HIP call, so that the hipGetLastError()
// after our own launch reports that launch only.
inline void clear_stale_hip_error() { (void)hipGetLastError(); }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SVDQ_OK;
  return set_error(SVDQ_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// `gemm`: the shape also runs the residual GEMM (the INT int32-accumulation bound applies)
int check_linear_dims(int64_t B, int64_t M, int64_t N, int64_t rank, int fmt, int bits, int dtype, bool gemm = true) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_format(fmt, bits))) return st;
  if (B < 1 || M < 1 || N < 1) return set_error(SVDQ_EINVAL, "B, M and N must be >= 1");
  if (B > kMaxDim || M > kMaxDim || N > kMaxDim) return set_error(SVDQ_EINVAL, "dimension too large");
  if (rank < 0 || rank > std::min(M, N)) return set_error(SVDQ_EINVAL, "rank must be in [0, min(M, N)]");
  return gemm ? check_int_accumulation(M, fmt, bits) : SVDQ_OK;
}

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" {

int svdq_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t rank, int fmt, int bits, int dtype,
                         size_t* bytes_out) {
  clear_error();
  int st = check_linear_dims(B, M, N, rank, fmt, bits, dtype, false);  // a size query (also for quantize_activations)
  if (st) return st;
  if (!bytes_out) return set_error(SVDQ_EINVAL, "bytes_out is NULL");
  const Dims d = make_dims(M, N, rank, fmt, bits, dtype);
  int64_t off[WS_NSEC];
  workspace_layout(d, make_plan(d, B), off);
  *bytes_out = (size_t)off[WS_END];
  return SVDQ_OK;
}

int svdq_smooth_inputs(const void* x, int64_t B, int64_t M, int64_t sxb, int64_t sxm, const void* weight, int64_t N,
                       int64_t swm, int64_t swn, const float* scale, int dtype, void* xs_out, int64_t ldxs,
                       void* ws_out, int64_t ldws, svdq_stream_t stream) {
  clear_error();
  clear_stale_hip_error();
  int st = check_dtype(dtype);
  if (st) return st;
  if (!scale) return set_error(SVDQ_EINVAL, "scale is NULL");
  if (M < 1 || M > kMaxDim) return set_error(SVDQ_EINVAL, "M must be >= 1");
  const bool do_x = x && xs_out, do_w = weight && ws_out;
  if (!do_x && !do_w) return set_error(SVDQ_EINVAL, "nothing to smooth");
  if (do_x && (B < 1 || B > kMaxDim || ldxs < M)) return set_error(SVDQ_EINVAL, "bad x shape or xs row stride");
  if (do_w && (N < 1 || N > kMaxDim || ldws < N)) return set_error(SVDQ_EINVAL, "bad weight shape or ws row stride");
  return hip_status(launch_smooth(do_x ? x : nullptr, B, M, sxb, sxm, do_w ? weight : nullptr, N, swm, swn, scale,
                                  dtype, do_x ? xs_out : nullptr, ldxs, do_w ? ws_out : nullptr, ldws,
                                  (hipStream_t)stream),
                    "smooth_inputs launch");
}

int svdq_calibrate_workspace_bytes(int64_t B, int64_t M, size_t* bytes_out) {
  clear_error();
  if (!bytes_out) return set_error(SVDQ_EINVAL, "bytes_out is NULL");
  if (B < 1 || B > kMaxDim || M < 1 || M > kMaxDim) return set_error(SVDQ_EINVAL, "B and M must be >= 1");
  *bytes_out = (size_t)round_up((int64_t)calib_parts(B, M) * M * 4, kAlign);
  return SVDQ_OK;
}

int svdq_calibrate_scale(const void* x, int64_t B, int64_t M, int64_t ldx, const void* weight, int64_t N, int64_t ldw,
                         int dtype, double alpha, float* scale_out, void* workspace, size_t workspace_bytes,
                         svdq_stream_t stream) {
  clear_error();
  clear_stale_hip_error();
  int st = check_dtype(dtype);
  if (st) return st;
  if (!x || !weight || !scale_out || !workspace) return set_error(SVDQ_EINVAL, "NULL buffer");
  if (B < 1 || B > kMaxDim || M < 1 || M > kMaxDim || N < 1 || N > kMaxDim)
    return set_error(SVDQ_EINVAL, "x [B,M] and weight [M,N] must be nonempty");
  if (ldx < M || ldw < N) return set_error(SVDQ_EINVAL, "row stride smaller than the row");
  if (!(alpha >= 0.0 && alpha <= 1.0)) return set_error(SVDQ_EINVAL, "alpha must be in [0, 1]");
  size_t need = 0;
  if ((st = svdq_calibrate_workspace_bytes(B, M, &need))) return st;
  if (workspace_bytes < need || !aligned(workspace, kAlign)) return set_error(SVDQ_EINVAL, "workspace too small or not 256-byte aligned");
  if (!aligned(x, dtype_size(dtype)) || !aligned(weight, dtype_size(dtype)) || !aligned(scale_out, 4))
    return set_error(SVDQ_EINVAL, "misaligned buffer");
  return hip_status(launch_calibrate(x, (int)B, (int)M, ldx, weight, (int)N, ldw, dtype, alpha, (float*)workspace,
                                     scale_out, (hipStream_t)stream),
                    "calibrate_scale launch");
}

size_t svdq_fake_quantize_workspace(int64_t rows, int64_t cols) {
  (void)cols;
  const int64_t parts = std::max<int64_t>(1, std::min<int64_t>(rows, 1024));
  return (size_t)round_up(parts * 4, kAlign);
}

int svdq_fake_quantize(const void* z, int64_t rows, int64_t cols, int64_t szr, int64_t szc, int dtype, int bits,
                       void* out, int64_t ldo, float* s_out, void* workspace, size_t workspace_bytes,
                       svdq_stream_t stream) {
  clear_error();
  clear_stale_hip_error();
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_format(SVDQ_FMT_INT, bits))) return st;
  if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim) return set_error(SVDQ_EINVAL, "empty or too large tensor");
  if (!z || !out || !workspace) return set_error(SVDQ_EINVAL, "NULL buffer");
  if (ldo < cols) return set_error(SVDQ_EINVAL, "output row stride smaller than cols");
  if (workspace_bytes < svdq_fake_quantize_workspace(rows, cols)) return set_error(SVDQ_EINVAL, "workspace too small");
  if (!aligned(workspace, 4)) return set_error(SVDQ_EINVAL, "workspace misaligned");
  const int parts = (int)std::min<int64_t>(rows, 1024);
  hipStream_t s = (hipStream_t)stream;
  float* part = (float*)workspace;
  if ((st = hip_status(launch_amax(z, rows, cols, szr, szc, nullptr, dtype, part, parts, s), "fake_quantize max"))) return st;
  return hip_status(launch_fake_quant(z, rows, cols, szr, szc, dtype, bits, part, parts, out, ldo, s_out, s),
                    "fake_quantize launch");
}

int svdq_quantize_activations(const void* x, int64_t B, int64_t M, int64_t ldx, const float* scale, int fmt, int bits,
                              int dtype, void* codes_out, int64_t ldc, void* scales_out, int64_t lds, float* sx_out,
                              void* workspace, size_t workspace_bytes, svdq_stream_t stream) {
  clear_error();
  clear_stale_hip_error();
  int st = check_linear_dims(B, M, 1, 0, fmt, bits, dtype, false);  // codes only, no residual GEMM
  if (st) return st;
  if (!x || !scale || !codes_out || !workspace) return set_error(SVDQ_EINVAL, "NULL buffer");
  if (fmt == SVDQ_FMT_MX && !scales_out) return set_error(SVDQ_EINVAL, "MX needs scales_out");
  const Dims d = make_dims(M, 1, 0, fmt, bits, dtype);
  if (ldx < M) return set_error(SVDQ_EINVAL, "x row stride smaller than M");
  if (ldc < d.code_row_bytes() || ldc % 16 || !aligned(codes_out, 16))
    return set_error(SVDQ_EINVAL, "codes_out must be 16-byte aligned with a row stride >= the padded width and a multiple of 16");
  if (fmt == SVDQ_FMT_MX && lds < d.mx_scale_row_bytes()) return set_error(SVDQ_EINVAL, "scale row stride too small");
  if (!aligned(scale, 16)) return set_error(SVDQ_EINVAL, "scale must be 16-byte aligned");
  const LaunchPlan pl = make_plan(d, B);
  int64_t off[WS_NSEC];
  workspace_layout(d, pl, off);
  if (workspace_bytes < (size_t)off[WS_END] || !aligned(workspace, kAlign))
    return set_error(SVDQ_EINVAL, "workspace too small or not 256-byte aligned");
  uint8_t* ws = (uint8_t*)workspace;
  hipStream_t s = (hipStream_t)stream;
  float* amax = (float*)(ws + off[WS_AMAX]);
  float* recip = (float*)(ws + off[WS_RECIP]);
  if ((st = hip_status(launch_reciprocals(scale, (int)M, recip, s), "reciprocal launch"))) return st;
  if (fmt == SVDQ_FMT_INT) {
    if ((st = hip_status(launch_amax_smoothed(x, (int)B, (int)M, ldx, scale, recip, dtype, amax, pl.amax_cols,
                                              pl.amax_rows, s),
                         "activation max")))
      return st;
  }
  ActParams p{};
  p.x = x;
  p.ldx = ldx;
  p.B = (int)B;
  p.M = (int)M;
  p.Kp = (int)d.Kp;
  p.scale = scale;
  p.recip = recip;
  p.codes = (uint8_t*)codes_out;
  p.ldc = ldc;
  p.mxs = (uint8_t*)scales_out;
  p.lds = lds;
  p.amax_part = amax;
  p.n_amax = pl.amax_blocks;
  p.bits = bits;
  p.sx_out = sx_out;
  p.l1t = nullptr;
  p.rp = 0;
  p.k_chunks = pl.k_chunks;
  p.k_chunk_len = pl.k_chunk_len;
  p.x_vec_ok = aligned(x, 16) && (ldx * (int64_t)dtype_size(dtype)) % 16 == 0;
  return hip_status(launch_act_quant(p, fmt, dtype, pl.row_blocks, 1, 64, s), "quantize_activations launch");
}

int svdq_linear(const void* x, int64_t B, int64_t M, int64_t ldx, const void* blob, int64_t N, int64_t rank, int fmt,
                int bits, int dtype, void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                svdq_stream_t stream) {
  return svdq_linear_bias(x, B, M, ldx, blob, N, rank, fmt, bits, dtype, nullptr, y, ldy, workspace, workspace_bytes,
                          stream);
}

int svdq_linear_bias(const void* x, int64_t B, int64_t M, int64_t ldx, const void* blob, int64_t N, int64_t rank,
                     int fmt, int bits, int dtype, const void* bias, void* y, int64_t ldy, void* workspace,
                     size_t workspace_bytes, svdq_stream_t stream) {
  clear_error();
  clear_stale_hip_error();
  int st = check_linear_dims(B, M, N, rank, fmt, bits, dtype);
  if (st) return st;
  if (bias && !aligned(bias, dtype_size(dtype))) return set_error(SVDQ_EINVAL, "bias misaligned");
  if (!x || !blob || !y || !workspace) return set_error(SVDQ_EINVAL, "NULL buffer");
  if (ldx < M) return set_error(SVDQ_EINVAL, "x row stride smaller than M");
  if (ldy < N) return set_error(SVDQ_EINVAL, "y row stride smaller than N");
  if (!aligned(blob, kAlign)) return set_error(SVDQ_EINVAL, "prepared blob must be 256-byte aligned");
  if (!aligned(y, dtype_size(dtype)) || !aligned(x, dtype_size(dtype))) return set_error(SVDQ_EINVAL, "x or y misaligned");
  const Dims d = make_dims(M, N, rank, fmt, bits, dtype);
  const LaunchPlan pl = make_plan(d, B);
  int64_t woff[WS_NSEC], boff[SVDQ_NSEC];
  workspace_layout(d, pl, woff);
  blob_layout(d, boff);
  if (workspace_bytes < (size_t)woff[WS_END] || !aligned(workspace, kAlign))
    return set_error(SVDQ_EINVAL, "workspace too small or not 256-byte aligned");
  const uint8_t* bl = (const uint8_t*)blob;
  uint8_t* ws = (uint8_t*)workspace;
  hipStream_t s = (hipStream_t)stream;
  float* amax = (float*)(ws + woff[WS_AMAX]);
  float* sx = (float*)(ws + woff[WS_SX]);
  const float* scale = (const float*)(bl + boff[SVDQ_SEC_SCALE]);
  const float* recip = (const float*)(bl + boff[SVDQ_SEC_RECIP]);

  const StageTimer tm(s);
  // (a) + (b): smooth, quantise, down-project
  if (fmt == SVDQ_FMT_INT) {
    tm.begin(0);
    if ((st = hip_status(launch_amax_smoothed(x, (int)B, (int)M, ldx, scale, recip, dtype, amax, pl.amax_cols,
                                              pl.amax_rows, s),
                         "activation max")))
      return st;
    tm.end(0);
  }
  ActParams p{};
  p.x = x;
  p.ldx = ldx;
  p.B = (int)B;
  p.M = (int)M;
  p.Kp = (int)d.Kp;
  p.scale = scale;
  p.recip = recip;
  p.codes = ws + woff[WS_CODES];
  p.ldc = d.code_row_bytes();
  p.mxs = ws + woff[WS_SCALES];
  p.lds = d.mx_scale_row_bytes();
  p.mxs_tiled = 1;
  p.amax_part = amax;
  p.n_amax = pl.amax_blocks;
  p.bits = bits;
  p.sx_out = sx;
  p.l1t = bl + boff[SVDQ_SEC_L1T];
  p.rp = (int)d.rp;
  p.down_part = (float*)(ws + woff[WS_PARTIAL]);
  p.down = ws + woff[WS_DOWN];
  p.k_chunks = pl.k_chunks;
  p.k_chunk_len = pl.k_chunk_len;
  p.x_vec_ok = aligned(x, 16) && (ldx * (int64_t)dtype_size(dtype)) % 16 == 0;
  const float* glob = (const float*)(bl + boff[SVDQ_SEC_GLOBAL]);  // {g_x, g_R, alpha, 0}
  if (fmt == SVDQ_FMT_MX) p.gscale = glob;
  // (c)'s parameters come first: the large-batch MXFP4 GEMM reads the activation codes in
  // 16-row tiles, which the activation kernel then writes
  GemmParams g{};
  g.acodes = ws + woff[WS_CODES];
  g.lda = d.code_row_bytes();
  g.ascales = ws + woff[WS_SCALES];
  g.ascale_groups = (int)ceil_div(B, 64);
  g.wcodes = bl + boff[SVDQ_SEC_RCODES];
  g.ldw = d.code_row_bytes();
  g.wscales = bl + boff[SVDQ_SEC_RSCALES];
  g.kq = (int)(d.Kp / 128);
  g.sx = sx;
  g.sr = (const float*)(bl + boff[SVDQ_SEC_RSCALES]);
  g.down = ws + woff[WS_DOWN];
  g.down_part = (const float*)(ws + woff[WS_PARTIAL]);  // split-K partials, summed by the GEMM epilogue
  g.down_chunks = pl.k_chunks;
  g.l2t = bl + boff[SVDQ_SEC_L2T];
  g.rp = (int)d.rp;
  g.y = y;
  g.bias = bias;
  if (fmt == SVDQ_FMT_MX) g.alpha = glob + 2;
  g.ldy = ldy;
  g.B = (int)B;
  g.N = (int)N;
  g.kstages = (int)(d.code_row_bytes() / 128);
  g.npad = (int)d.Np;
  if (fmt == SVDQ_FMT_MX && B > 64) {
    g.kstages = (int)(d.code_row_bytes() / 64);
    g.acodes_tiled = mx_large_accepts(g) ? 1 : 0;
    g.kstages = (int)(d.code_row_bytes() / 128);
  }
  if (fmt == SVDQ_FMT_MX && B <= 64) g.acodes_tiled = 1;  // the decode GEMM takes every such batch
  p.codes_tiled = g.acodes_tiled;
  tm.begin(1);
  if ((st = hip_status(launch_act_quant(p, fmt, dtype, pl.row_blocks, pl.r_chunks, pl.rchunk, s), "activation quantise launch")))
    return st;
  tm.end(1);
  tm.gemm_begin();
  hipError_t ge = hipErrorNotSupported;
  if (fmt == SVDQ_FMT_MX) {
    g.kstages = (int)(d.code_row_bytes() / 64);  // 64-byte stages
    ge = B <= 64 ? launch_gemm_mx_decode(g, dtype, s) : launch_gemm_mx_large(g, dtype, s);
    if (ge == hipErrorNotSupported && g.acodes_tiled) return set_error(SVDQ_EHIP, "tiled activation codes left without their GEMM");
    if (ge == hipErrorNotSupported) g.kstages = (int)(d.code_row_bytes() / 128);
  }
  if (fmt == SVDQ_FMT_INT) {
    g.kstages = (int)(d.code_row_bytes() / 128);  // 128-byte stages (256 codes)
    ge = launch_gemm_int_big(g, bits, dtype, s);
    if (ge == hipErrorNotSupported) ge = launch_gemm_int4(g, bits, dtype, s);
  }
  if (ge == hipErrorNotSupported) ge = launch_gemm(g, fmt, bits, dtype, s);
  tm.gemm_end(ge);
  st = hip_status(ge, "residual GEMM launch");
  return st;
}

// ---- svdq_linear_noalloc: svdq_linear with a library-owned scratch instead of a workspace.
// The scratch is one file-scope device array per GPU (each device holds its own copy from the
// moment the library's code object is loaded until the process ends). In host code `scratch`
// names a host-side stand-in, never the device memory: the device address is looked up once
// per device with hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
}  // extern "C"

static __device__ __align__(256) uint8_t scratch[SVDQ_NOALLOC_SCRATCH_BYTES];

namespace svdq {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // per-device address of `scratch`, or null

// Device address of this device's scratch (the current device, which the stream must belong
// to); looked up on the first call on each device. Concurrent first calls look it up twice
// and store the same address.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_error(SVDQ_EUNSUPPORTED, "device index above 63");
  hipDevice_t sdev = -1;
  if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return hip_status(e, "hipStreamGetDevice");
  if ((int)sdev != dev) return set_error(SVDQ_EINVAL, "the stream belongs to another device than the current one");
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    if ((e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch))) != hipSuccess) return hip_status(e, "hipGetSymbolAddress");
    if (!a || !aligned(a, kAlign)) return set_error(SVDQ_EHIP, "scratch symbol has no aligned device address");
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *out = a;
  return SVDQ_OK;
}
}  // namespace
}  // namespace svdq

extern "C" {

int svdq_linear_noalloc(const void* x, int64_t B, int64_t M, int64_t ldx, const void* blob, int64_t N, int64_t rank,
                        int fmt, int bits, int dtype, void* y, int64_t ldy, svdq_stream_t stream) {
  clear_error();
  int st = check_linear_dims(B, M, N, rank, fmt, bits, dtype);
  if (st) return st;
  const Dims d = make_dims(M, N, rank, fmt, bits, dtype);
  int64_t woff[WS_NSEC];
  workspace_layout(d, make_plan(d, B), woff);
  if (woff[WS_END] > (int64_t)SVDQ_NOALLOC_SCRATCH_BYTES)
    return set_error(SVDQ_EINVAL, "svdq_linear_noalloc: this shape needs " + std::to_string(woff[WS_END]) +
                                      " bytes of scratch, above its maximum of " +
                                      std::to_string((int64_t)SVDQ_NOALLOC_SCRATCH_BYTES) +
                                      " (use svdq_linear with a caller workspace)");
  void* ws = nullptr;
  if ((st = scratch_address((hipStream_t)stream, &ws))) return st;
  return svdq_linear_bias(x, B, M, ldx, blob, N, rank, fmt, bits, dtype, nullptr, y, ldy, ws,
                          (size_t)SVDQ_NOALLOC_SCRATCH_BYTES, stream);
}

int svdq_profile_begin(int max_calls, unsigned stage_mask) { return svdq_profile_begin_sampled(max_calls, stage_mask, 1); }

int svdq_profile_begin_sampled(int max_calls, unsigned stage_mask, int every) {
  clear_error();
  if (max_calls < 1) return set_error(SVDQ_EINVAL, "max_calls must be >= 1");
  if (every < 1) return set_error(SVDQ_EINVAL, "every must be >= 1");
  if (stage_mask == 0 || (stage_mask >> SVDQ_NSTAGES)) return set_error(SVDQ_EINVAL, "stage_mask must select stages 0..3");
  if (g_prof.open) return set_error(SVDQ_EINVAL, "a profiling session is already open");
  const size_t nev = (size_t)max_calls * SVDQ_NSTAGES * 2;
  g_prof.ev = new hipEvent_t[nev]();
  for (size_t i = 0; i < nev; i++) {
    hipError_t r = hipEventCreate(&g_prof.ev[i]);
    if (r != hipSuccess) {
      for (size_t j = 0; j < i; j++) hipEventDestroy(g_prof.ev[j]);
      delete[] g_prof.ev;
      g_prof.ev = nullptr;
      return hip_status(r, "hipEventCreate");
    }
  }
  g_prof.recorded = new uint8_t[(size_t)max_calls * SVDQ_NSTAGES]();
  g_prof.open = true;
  g_prof.mask = stage_mask;
  g_prof.max_calls = max_calls;
  g_prof.calls = 0;
  g_prof.every = every;
  g_prof.seen = 0;
  return SVDQ_OK;
}

int svdq_ceiling(int kind, int64_t arg, const void* buf, size_t buf_bytes, float* out, size_t out_bytes,
                 svdq_stream_t stream, double* work_out) {
  clear_error();
  clear_stale_hip_error();
  if (kind < 0 || kind > 2) return set_error(SVDQ_EINVAL, "kind must be 0 (FP4 MFMA), 1 (INT8 MFMA) or 2 (read stream)");
  if (!out || !work_out) return set_error(SVDQ_EINVAL, "NULL buffer");
  if (!aligned(out, 4)) return set_error(SVDQ_EINVAL, "misaligned buffer");
  double work = 0.0;
  const hipError_t e = launch_ceiling(kind, arg, buf, buf_bytes, out, out_bytes, (hipStream_t)stream, &work);
  if (e == hipErrorInvalidValue)
    return set_error(SVDQ_EINVAL, "iterations or blocks out of range, or a buffer too small or misaligned");
  if (e == hipSuccess) *work_out = work;
  return hip_status(e, "ceiling launch");
}

int svdq_profile_end(float* ms, int cap, int* n_calls) {
  clear_error();
  if (!g_prof.open) return set_error(SVDQ_EINVAL, "no profiling session is open");
  const int n = std::min(g_prof.calls, cap);
  for (int c = 0; c < n; c++) {
    for (int k = 0; k < SVDQ_NSTAGES; k++) {
      hipEvent_t a = g_prof.ev[((size_t)c * SVDQ_NSTAGES + k) * 2], b = g_prof.ev[((size_t)c * SVDQ_NSTAGES + k) * 2 + 1];
      float v = 0.f;
      if (g_prof.recorded[(size_t)c * SVDQ_NSTAGES + k]) {
        hipError_t r = hipEventSynchronize(b);
        if (r == hipSuccess) r = hipEventElapsedTime(&v, a, b);
        if (r != hipSuccess) v = 0.f;
      }
      if (ms) ms[(size_t)c * SVDQ_NSTAGES + k] = v;
    }
  }
  const size_t nev = (size_t)g_prof.max_calls * SVDQ_NSTAGES * 2;
  for (size_t i = 0; i < nev; i++) hipEventDestroy(g_prof.ev[i]);
  delete[] g_prof.ev;
  delete[] g_prof.recorded;
  g_prof.ev = nullptr;
  g_prof.recorded = nullptr;
  g_prof.open = false;
  clear_stale_hip_error();
  if (n_calls) *n_calls = n;
  return SVDQ_OK;
}

}  // extern "C"
