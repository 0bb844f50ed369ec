// Activation-side kernels of libsvdq for gfx950:
//   * k_smooth      — smooth_inputs, elementwise (x / scale, scale * W);
//   * k_amax_part   — per-block maxima of |z| or |x / scale| (per-tensor INT pre-pass);
//   * k_fake_quant  — per-tensor INT fake quantisation (dequantised values);
//   * k_act_quant   — step (a)+(b) of the operator: X^ = D(x / scale), its INT or MXFP4
//                     codes, and the low-rank down-projection X^ L1 on the matrix cores;
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization" ("Formula and
// conventions" items 1 and 3: smoothing divides x by scale; the low-rank branch takes the
// unquantised smoothed activations; per-tensor INT with ties to even) and the msModelSlim
// SVDQuant guide, step 2 (MXFP4 per-block minmax activations).
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

// ------------------------------------------------------------------------- smooth_inputs
template <class DT>
__global__ void k_smooth_x(const typename DT::T* __restrict__ x, int64_t B, int64_t M, int64_t sxb, int64_t sxm,
                           const float* __restrict__ scale, typename DT::T* __restrict__ xs, int64_t ldxs) {
  const int64_t n = B * M;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / M, m = i - b * M;
    const float v = DT::to_f32(x[b * sxb + m * sxm]), s = scale[m];
    if constexpr (DT::is_bf16) {
      // the same rounding path as the operator's activation kernel
      const float y = (s >= 0x1p-90f && s <= 0x1p90f) ? 1.0f / s : 0.f;
      xs[b * ldxs + m] = DT::from_f32(smooth_bf16(v, s, y));
    } else {
      xs[b * ldxs + m] = DT::from_f32(v / s);
    }
  }
}

template <class DT>
__global__ void k_smooth_w(const typename DT::T* __restrict__ w, int64_t M, int64_t N, int64_t swm, int64_t swn,
                           const float* __restrict__ scale, typename DT::T* __restrict__ ws, int64_t ldws) {
  const int64_t n = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / N, j = i - m * N;
    ws[m * ldws + j] = DT::from_f32(scale[m] * DT::to_f32(w[m * swm + j * swn]));
  }
}

// ------------------------------------------------------------------------- block max helper
// Max over the 256 threads of a block; every thread receives the result.
__device__ inline float block_max256(float v, float* sh) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

// Max of part[0..n) computed by the whole block (max is exact and order-free).
__device__ inline float reduce_parts(const float* __restrict__ part, int n, float* sh) {
  float a = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) a = fmaxf(a, part[i]);
  return block_max256(a, sh);
}

// ------------------------------------------------------------------------- per-tensor max
// Block p covers rows [p*rpb, (p+1)*rpb); threads stride over the columns of each row.
template <class DT, bool SMOOTH>
__global__ __launch_bounds__(256) void k_amax_part(const typename DT::T* __restrict__ z, int64_t rows, int64_t cols,
                                                   int64_t szr, int64_t szc, const float* __restrict__ scale,
                                                   float* __restrict__ part) {
  __shared__ float sh[4];
  const int64_t rpb = (rows + gridDim.x - 1) / gridDim.x;
  const int64_t r0 = (int64_t)blockIdx.x * rpb, r1 = r0 + rpb < rows ? r0 + rpb : rows;
  float a = 0.f;
  for (int64_t r = r0; r < r1; r++) {
    for (int64_t c = threadIdx.x; c < cols; c += 256) {
      float v = DT::to_f32(z[r * szr + c * szc]);
      if (SMOOTH) v = smooth_value<DT>(v, scale[c]);
      a = fmaxf(a, fabsf(v));
    }
  }
  a = block_max256(a, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = a;
}

// ------------------------------------------------------------------------- fake_quantize
template <class DT>
__global__ __launch_bounds__(256) void k_fake_quant(const typename DT::T* __restrict__ z, int64_t rows, int64_t cols,
                                                    int64_t szr, int64_t szc, int bits, const float* __restrict__ part,
                                                    int nparts, typename DT::T* __restrict__ out, int64_t ldo,
                                                    float* __restrict__ s_out) {
  __shared__ float sh[4];
  const float amax = reduce_parts(part, nparts, sh);
  const float qmax = (float)((1 << (bits - 1)) - 1);
  const float s = amax / qmax;  // IEEE division; 0 for an all-zero tensor
  if (blockIdx.x == 0 && threadIdx.x == 0 && s_out) *s_out = s;
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    const int code = int_code(DT::to_f32(z[r * szr + c * szc]), s, qmax);
    out[r * ldo + c] = DT::from_f32(s * (float)code);
  }
}

// ------------------------------------------------------------------------- per-tensor max of X^
// max_{b,m} |D(x[b,m] / scale[m])| = max_m D(max_b |x[b,m]| / scale[m]): division by a positive
// scale and rounding to the dtype are monotone, so each block takes column maxima of |x| over
// its rows (one max per element) and divides once per column. Block (cx, ry): columns
// [2048 cx, 2048 cx + 2048) (8 per thread), rows [rpb ry, rpb ry + rpb).
template <class DT>
__global__ __launch_bounds__(256) void k_amax_cols(const typename DT::T* __restrict__ x, int B, int M, int64_t ldx,
                                                   const float* __restrict__ scale, const float* __restrict__ recip,
                                                   int rpb, int vec_ok, float* __restrict__ part) {
  __shared__ float sh[4];
  const int c0 = blockIdx.x * 2048 + threadIdx.x * 8;
  const int r0 = blockIdx.y * rpb, r1 = r0 + rpb < B ? r0 + rpb : B;
  // this thread's scales and reciprocals, loaded together with x (one memory round trip)
  float sc8[8], rc8[8];
#pragma unroll
  for (int q = 0; q < 8; q++) {
    sc8[q] = 1.f;
    rc8[q] = 0.f;
  }
  if (c0 + 8 <= M) {
    const float4 s0 = *reinterpret_cast<const float4*>(scale + c0), s1 = *reinterpret_cast<const float4*>(scale + c0 + 4);
    const float4 y0 = *reinterpret_cast<const float4*>(recip + c0), y1 = *reinterpret_cast<const float4*>(recip + c0 + 4);
    sc8[0] = s0.x; sc8[1] = s0.y; sc8[2] = s0.z; sc8[3] = s0.w; sc8[4] = s1.x; sc8[5] = s1.y; sc8[6] = s1.z; sc8[7] = s1.w;
    rc8[0] = y0.x; rc8[1] = y0.y; rc8[2] = y0.z; rc8[3] = y0.w; rc8[4] = y1.x; rc8[5] = y1.y; rc8[6] = y1.z; rc8[7] = y1.w;
  } else {
    for (int q = 0; q < 8 && c0 + q < M; q++) {
      sc8[q] = scale[c0 + q];
      rc8[q] = recip[c0 + q];
    }
  }
  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < M) {
    int r = r0;
    if (DT::is_bf16 && vec_ok && c0 + 8 <= M) {
      // rounds of U rows (8 while they last, then 4, 2, 1), all loads issued before the maxima
      auto rows = [&](auto uc) {
        constexpr int U = decltype(uc)::value;
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; u++) w[u] = *reinterpret_cast<const uint4*>(x + (int64_t)(r + u) * ldx + c0);
#pragma unroll
        for (int u = 0; u < U; u++) {
          const u32 ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
          for (int h = 0; h < 4; h++) {
            cm[2 * h] = fmaxf(cm[2 * h], fabsf(__uint_as_float(ws[h] << 16)));
            cm[2 * h + 1] = fmaxf(cm[2 * h + 1], fabsf(__uint_as_float(ws[h] & 0xFFFF0000u)));
          }
        }
        r += U;
      };
      while (r + 8 <= r1) rows(std::integral_constant<int, 8>());
      if (r + 4 <= r1) rows(std::integral_constant<int, 4>());
      if (r + 2 <= r1) rows(std::integral_constant<int, 2>());
      if (r < r1) rows(std::integral_constant<int, 1>());
    }
    for (; r < r1; r++) {
      const typename DT::T* xr = x + (int64_t)r * ldx + c0;
      if (vec_ok && c0 + 8 <= M) {
        if constexpr (DT::is_bf16) {
          const uint4 w = *reinterpret_cast<const uint4*>(xr);
          const u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int h = 0; h < 4; h++) {
            cm[2 * h] = fmaxf(cm[2 * h], fabsf(__uint_as_float(ws[h] << 16)));
            cm[2 * h + 1] = fmaxf(cm[2 * h + 1], fabsf(__uint_as_float(ws[h] & 0xFFFF0000u)));
          }
        } else {
          const float4 a = *reinterpret_cast<const float4*>(xr), b = *reinterpret_cast<const float4*>(xr + 4);
          const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
          for (int q = 0; q < 8; q++) cm[q] = fmaxf(cm[q], fabsf(v[q]));
        }
      } else {
        for (int q = 0; q < 8 && c0 + q < M; q++) cm[q] = fmaxf(cm[q], fabsf(DT::to_f32(xr[q])));
      }
    }
  }
  float a = 0.f;
#pragma unroll
  for (int q = 0; q < 8; q++)
    if (c0 + q < M) a = fmaxf(a, DT::to_f32(DT::from_f32(div_rn(cm[q], sc8[q], rc8[q]))));
  a = block_max256(a, sh);
  if (threadIdx.x == 0) part[blockIdx.y * gridDim.x + blockIdx.x] = a;
}

// ------------------------------------------------------------------------- step (a) + (b)
// Block (rb, kc, rc): rows [16 rb, 16 rb + 16), K range [kc * k_chunk_len, ...), low-rank
// columns [64 rc, 64 rc + 64). Eight waves walk the K range in 128-wide steps. In a step,
// lane l owns row l % 16 and the whole 32-element block l / 16 of that step: the block max,
// shared exponent and codes stay inside the lane. For the down-projection the lane feeds the
// same 32 values to the matrix cores: 16x16x32 bf16 MFMAs in four K-slices of 8 (the B
// operand lane (n, g) supplies L1^T[n] at the same K offsets, so the K order is consistent).
// L1^T is stored in 16-row x 128-K tiles ordered by (K-slice, block, row), so the B operand of
// one MFMA is a single contiguous 1 KB wave load.
//
// Steps that lie wholly inside [0, M) with 16-byte aligned rows run a branch-free body (all
// of the step's loads are independent and issue together); only the tail step and the zero
// padding up to Kp take the guarded body.
constexpr int ACT_WAVES = 8;
// Low-rank columns per block (RC, a template parameter of the kernel): 64, or 16 when rows x
// rank chunks would give too few blocks (decode-sized batches); the 16-wide form repeats the
// smoothing of its K range for each rank chunk, which is cheap next to the parallelism won.

template <class DT>
__device__ inline void load_row32(const typename DT::T* __restrict__ xrow, int k, int M, bool vec_ok, u32* raw) {
  // raw: the 32 values as stored (bf16: 16 words of pairs; f32: 32 words)
  constexpr int W = DT::is_bf16 ? 16 : 32;
  if (vec_ok && k + 32 <= M) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow + k);
#pragma unroll
    for (int q = 0; q < W / 4; q++) {
      const uint4 w = src[q];
      raw[4 * q] = w.x;
      raw[4 * q + 1] = w.y;
      raw[4 * q + 2] = w.z;
      raw[4 * q + 3] = w.w;
    }
  } else {
    if constexpr (DT::is_bf16) {
#pragma unroll
      for (int h = 0; h < 16; h++) {
        const u32 lo = (k + 2 * h < M) ? (u32)xrow[k + 2 * h] : 0u;
        const u32 hi = (k + 2 * h + 1 < M) ? (u32)xrow[k + 2 * h + 1] : 0u;
        raw[h] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; j++) raw[j] = (k + j < M) ? __float_as_uint(xrow[k + j]) : 0u;
    }
  }
}

// n consecutive floats of a per-channel array (scale or reciprocal); `pad` past M unless FULL.
template <bool FULL>
__device__ inline void load_chan(const float* __restrict__ a, int k, int M, float pad, float* v) {
  if (FULL) {
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const float4 u = *reinterpret_cast<const float4*>(a + k + 4 * q);
      v[4 * q] = u.x; v[4 * q + 1] = u.y; v[4 * q + 2] = u.z; v[4 * q + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; j++) v[j] = (k + j < M) ? a[k + j] : pad;
  }
}

// Per-lane constants of a block.
struct ActLane {
  int lane, i, g, b, rbase, nbl;
  int xoff[4];  // full bf16 steps: element offsets (from the block's first row) of the lane's four x loads
  bool do_codes;
  float sx, ysx, qmax;
  float gx;  // MX two-level scaling: codes of RN(X^ g_x) (1 when not scaled)
};

// Broadcast of lane Q of each 16-lane row to the whole row (DPP row_newbcast; the compiler
// folds it into the consuming VALU instruction).
template <int Q>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + Q, 0xF, 0xF, false));
}

// The step's B operands of the down-projection (bf16 L1^T, tiled 16 rank columns x 128 K per
// 2048 elements): lane (i, g) takes four 16-byte pieces per 16-column tile.
template <int RC, class T>
__device__ __forceinline__ void load_l1(const ActParams& p, const ActLane& L, int k0, v4i (&bw)[RC / 16][4]) {
  const T* __restrict__ l1t = reinterpret_cast<const T*>(p.l1t);
#pragma unroll
  for (int n = 0; n < RC / 16; n++)
    if (n < L.nbl) {
      const T* tile = l1t + ((int64_t)(L.rbase / 16 + n) * (p.Kp / 128) + k0 / 128) * 2048 + L.lane * (16 / sizeof(T));
#pragma unroll
      for (int c = 0; c < 4; c++) bw[n][c] = *reinterpret_cast<const v4i*>(tile + c * 512);
    }
}

// The same for the full steps of a block with low-rank columns (nbl >= 1), with a fixed number
// of loads: tiles past the block's last (only in a partial 64-wide chunk) reload that one, their
// operands unused. The compiler counts the loads issued after an operand to wait for it alone;
// a conditional load would make that count unknown and the wait cover every later load, the
// next step's prefetch included.
template <int RC, class T>
__device__ __forceinline__ void load_l1_all(const ActParams& p, const ActLane& L, int k0, v4i (&bw)[RC / 16][4]) {
  const T* __restrict__ l1t = reinterpret_cast<const T*>(p.l1t);
#pragma unroll
  for (int n = 0; n < RC / 16; n++) {
    const int tn = n < L.nbl ? n : L.nbl - 1;
    const T* tile = l1t + ((int64_t)(L.rbase / 16 + tn) * (p.Kp / 128) + k0 / 128) * 2048 + L.lane * (16 / sizeof(T));
#pragma unroll
    for (int c = 0; c < 4; c++) bw[n][c] = *reinterpret_cast<const v4i*>(tile + c * 512);
  }
}

// Whether a full step's L1^T operands travel one step ahead with its x: with 16 or 32 rank
// columns per block (16 or 32 registers per step in flight). The 64-wide form would run out of
// registers: it requests the current step's operands at the top of the step, before the next
// step's x. (Loads return in issue order, so the wait for an operand also waits for every
// load issued before it: operands requested after the next step's x would make every step
// wait for that x, a full HBM round trip.)
constexpr bool l1_ahead(int RC) { return RC <= 32; }

// Inputs of a full bf16 step that the caller loads one step ahead: 16 words of bf16 x pairs as
// the quad loads left them (quad_transpose turns them into the lane's own 32 values), two
// reciprocals and two scales, and (l1_ahead) the step's L1^T operands. Lane l = 16 g + q holds
// RN(1/s) and s of columns k0 + 2 l and k0 + 2 l + 1, i.e. the pair q of the block that the
// lanes of row g work on.
template <int RC>
struct FullIn {
  u32 raw[16];
  float2 y2, s2;
  v4i bw[l1_ahead(RC) ? RC / 16 : 1][4];
};

// x of a full step, loaded by quads: in load q, the quad j of a 16-lane row g (lanes 4j..4j+3)
// reads the 64 contiguous bytes of block g in row 4j + q, lane 4j + t taking the 16-byte piece
// t. So each load covers 4 rows x 256 contiguous bytes (8 cache lines) instead of 16 rows x 4
// scattered pieces (32 lines). Lane 4j + t then holds piece t of rows 4j..4j+3 and needs pieces
// 0..3 of row 4j + t: a 4 x 4 transpose of (lane in quad, load) done by quad_transpose at use.
template <int RC, bool LR, class T>
__device__ __forceinline__ void load_full(const ActParams& p, const T* __restrict__ xblk, const ActLane& L, int k0,
                                          FullIn<RC>& in) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint4 w = *reinterpret_cast<const uint4*>(xblk + (L.xoff[q] + k0));
    in.raw[4 * q] = w.x; in.raw[4 * q + 1] = w.y; in.raw[4 * q + 2] = w.z; in.raw[4 * q + 3] = w.w;
  }
  in.y2 = *reinterpret_cast<const float2*>(p.recip + k0 + 2 * L.lane);
  in.s2 = *reinterpret_cast<const float2*>(p.scale + k0 + 2 * L.lane);
  if constexpr (l1_ahead(RC) && LR) load_l1_all<RC, T>(p, L, k0, in.bw);
}

// The 4 x 4 transpose of load_full's pieces within each quad of lanes: afterwards lane t of a quad
// holds in word 4 p + d what lane p held in word 4 t + d. Two butterfly rounds (lane and piece
// bit 1, then bit 0), each swapping one word per piece pair with the partner lane (DPP
// quad_perm, whole wave active).
struct RawStep {
  u32 raw[16];
  float2 y2, s2;
};
// One butterfly round of quad_transpose: lanes and pieces whose bit M differ trade words.
template <int M>
__device__ __forceinline__ void quad_swap_round(u32 (&a)[16], int t) {
  constexpr int CTRL = M == 2 ? 0x4E : 0xB1;  // quad_perm [2,3,0,1] or [1,0,3,2]
  const bool hm = (t & M) != 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if (q & M) continue;
#pragma unroll
    for (int d = 0; d < 4; d++) {
      // the partner's words of both pieces; a lane with bit M takes the partner's piece q | M
      // in place of its piece q, a lane without it the partner's piece q in place of q | M
      const u32 lo = a[4 * q + d], hi = a[4 * (q | M) + d];
      const u32 p_hi = (u32)__builtin_amdgcn_mov_dpp((int)hi, CTRL, 0xF, 0xF, true);
      const u32 p_lo = (u32)__builtin_amdgcn_mov_dpp((int)lo, CTRL, 0xF, 0xF, true);
      a[4 * q + d] = hm ? p_hi : lo;
      a[4 * (q | M) + d] = hm ? hi : p_lo;
    }
  }
}
template <int RC>
__device__ __forceinline__ void quad_transpose(const FullIn<RC>& in, int lane, RawStep& out) {
  u32 a[16];
#pragma unroll
  for (int w = 0; w < 16; w++) a[w] = in.raw[w];
  quad_swap_round<2>(a, lane & 3);
  quad_swap_round<1>(a, lane & 3);
#pragma unroll
  for (int w = 0; w < 16; w++) out.raw[w] = a[w];
  out.y2 = in.y2;
  out.s2 = in.s2;
}

// Full bf16 steps, exact path: X^ = RN_bf16(RN_f32(x / s)) for every element by div_markstein,
// with the reciprocal and the scale of each column broadcast from the lane that loaded them
// (DPP, while the whole wave is active); an overflowing quotient shows up as a bf16 NaN and is
// replaced by +-infinity afterwards (a wave-uniform branch that real data never takes).
// amax16 keeps max |X^| as bf16 bit patterns in two 16-bit lanes (for non-negative values the
// integer order is the numeric order).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int Q, class IN>
__device__ __forceinline__ void exact_pair(const IN& in, u32* xb, u16x2& amax16) {
  const float x0 = __uint_as_float(in.raw[Q] << 16), x1 = __uint_as_float(in.raw[Q] & 0xFFFF0000u);
  const float t0 = div_markstein(x0, row_bcast<Q>(in.s2.x), row_bcast<Q>(in.y2.x));
  const float t1 = div_markstein(x1, row_bcast<Q>(in.s2.y), row_bcast<Q>(in.y2.y));
  const u32 pk = pack_bf16x2(t0, t1);
  xb[Q] = pk;
  amax16 = __builtin_elementwise_max(amax16, __builtin_bit_cast(u16x2, pk & 0x7FFF7FFFu));
}
template <class IN, int... Q>
__device__ __forceinline__ void exact_pairs(std::integer_sequence<int, Q...>, const IN& in, u32* xb, u16x2& amax16) {
  (exact_pair<Q>(in, xb, amax16), ...);
}

// Pair Q by the fast product: t = RN(x * RN(1/s)) is within 2 f32 ulps of RN_f32(x / s), so
// RN_bf16(t) is the exact result unless t's low 16 bits lie within 3 of the bf16 rounding
// midpoint 0x8000. Those low halves are gathered in pairs and their distance to the band
// kept as a running minimum (packed 16-bit ops); the caller redoes the step exactly when any
// lane of the wave saw one. (Products that underflow or overflow need no special case: near
// zero the f32 error is far below the bf16 spacing, past the bf16 range both give inf.)
template <int Q, class IN>
__device__ __forceinline__ void fast_pair(const IN& in, u32* xb, u16x2& amax16, u16x2& band) {
  const float x0 = __uint_as_float(in.raw[Q] << 16), x1 = __uint_as_float(in.raw[Q] & 0xFFFF0000u);
  const float t0 = x0 * row_bcast<Q>(in.y2.x), t1 = x1 * row_bcast<Q>(in.y2.y);
  const u32 pk = pack_bf16x2(t0, t1);
  xb[Q] = pk;
  amax16 = __builtin_elementwise_max(amax16, __builtin_bit_cast(u16x2, pk & 0x7FFF7FFFu));
  const u32 lows = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x05040100u);
  band = __builtin_elementwise_min(band, __builtin_bit_cast(u16x2, lows) + (u16x2){0x8003, 0x8003});
}
template <class IN, int... Q>
__device__ __forceinline__ void fast_pairs(std::integer_sequence<int, Q...>, const IN& in, u32* xb, u16x2& amax16,
                                           u16x2& band) {
  (fast_pair<Q>(in, xb, amax16, band), ...);
}

// Replace bf16 NaNs (quotients that overflowed) by infinity with the sign of x.
__device__ __forceinline__ u32 nan_to_inf_pair(u32 pk, u32 raw) {
  u32 r = pk;
  if ((pk & 0x7FFFu) > 0x7F80u) r = (r & 0xFFFF0000u) | 0x7F80u | ((raw >> 0) & 0x8000u);
  if ((pk & 0x7FFF0000u) > 0x7F800000u) r = (r & 0x0000FFFFu) | 0x7F800000u | (raw & 0x80000000u);
  return r;
}

// State a step carries from its smoothing half to its codes + down-projection half: X^ as
// stored (bf16 pairs or f32 bits), max |X^| of the lane's block, and (bf16) the step's L1^T
// operands.
template <class DT, int RC>
struct StepState {
  u32 xb[DT::is_bf16 ? 16 : 32];
  float amax;
  v4i bw[RC / 16][4];
};

// First half of a step: loads, X^ = D(x / scale) and its block maximum.
template <class DT, int FMT, bool NIB, bool FULL, int RC>
__device__ __forceinline__ void act_smooth(const ActParams& p, const typename DT::T* __restrict__ xrow, const ActLane& L,
                                           int k0, const FullIn<RC>& in_q, const v4i (&bwc)[RC / 16][4],
                                           StepState<DT, RC>& st) {
  typedef typename DT::T T;
  constexpr int RW = DT::is_bf16 ? 16 : 32;
  constexpr bool FAST = DT::is_bf16 && FULL;
  const int k = k0 + 32 * L.g;
  const T* __restrict__ l1t = reinterpret_cast<const T*>(p.l1t);
  u32* xb = st.xb;
  auto& bw = st.bw;

  u32 raw[RW];
  float s32[32], y32[32];
  if constexpr (!FAST) {
    if (FULL) {
      const uint4* src = reinterpret_cast<const uint4*>(xrow + k);
#pragma unroll
      for (int q = 0; q < RW / 4; q++) {
        const uint4 w = src[q];
        raw[4 * q] = w.x; raw[4 * q + 1] = w.y; raw[4 * q + 2] = w.z; raw[4 * q + 3] = w.w;
      }
    } else {
      load_row32<DT>(xrow, k, p.M, p.x_vec_ok, raw);
    }
    load_chan<FULL>(p.scale, k, p.M, 1.f, s32);
    load_chan<FULL>(p.recip, k, p.M, 1.f, y32);
  }
  // B operands of the down-projection for this step (bf16: with l1_ahead full steps got them
  // one step ahead with x, other full steps at the top of the step (bwc), the remaining steps
  // load them with their other loads; f32 loads them at the MFMAs to save registers)
  constexpr int NB = RC / 16;
  if constexpr (FAST && l1_ahead(RC)) {
#pragma unroll
    for (int n = 0; n < NB; n++)
#pragma unroll
      for (int c = 0; c < 4; c++) bw[n][c] = in_q.bw[n][c];
  } else if constexpr (FAST) {
#pragma unroll
    for (int n = 0; n < NB; n++)
#pragma unroll
      for (int c = 0; c < 4; c++) bw[n][c] = bwc[n][c];
  } else if (DT::is_bf16 && L.nbl > 0) {
    load_l1<RC, T>(p, L, k0, bw);
  }

  // X^ = D(x / scale); xb: X^ as stored (bf16 pairs or f32 bits); amax: max |X^| before the
  // final rounding to the dtype (rounding is monotone, so it rounds to max |X^|).
  float amax = 0.f;
  if constexpr (FAST) {
    RawStep tin;
    quad_transpose(in_q, L.lane, tin);
    const RawStep& in = tin;
    u16x2 amax16 = {0, 0};
    if (__all(in.y2.x != 0.f && in.y2.y != 0.f)) {
      u16x2 band = {0xFFFF, 0xFFFF};
      fast_pairs(std::make_integer_sequence<int, 16>{}, in, xb, amax16, band);
      // a product near a midpoint, or a NaN, anywhere in the wave: the whole step exactly
      const bool redo = (band.x < 7 || band.y < 7) || (amax16.x > amax16.y ? amax16.x : amax16.y) > 0x7F80;
      if (__any(redo)) {
        amax16 = (u16x2){0, 0};
        exact_pairs(std::make_integer_sequence<int, 16>{}, in, xb, amax16);
      }
      if (__any((amax16.x > amax16.y ? amax16.x : amax16.y) > 0x7F80)) {
        // an overflowing quotient somewhere in the wave (never for real activations)
        amax16 = (u16x2){0, 0};
#pragma unroll
        for (int q = 0; q < 16; q++) {
          xb[q] = nan_to_inf_pair(xb[q], in.raw[q]);
          amax16 = __builtin_elementwise_max(amax16, __builtin_bit_cast(u16x2, xb[q] & 0x7FFF7FFFu));
        }
      }
    } else {
      // a stored reciprocal of 0 (scale outside [2^-90, 2^90]) among these columns: per-element rule
#pragma unroll
      for (int j = 0; j < 32; j += 2) {
        const float x0 = __uint_as_float(in.raw[j / 2] << 16), x1 = __uint_as_float(in.raw[j / 2] & 0xFFFF0000u);
        const float t0 = smooth_bf16(x0, p.scale[k + j], p.recip[k + j]);
        const float t1 = smooth_bf16(x1, p.scale[k + j + 1], p.recip[k + j + 1]);
        const u32 pk = pack_bf16x2(t0, t1);
        xb[j / 2] = pk;
        amax16 = __builtin_elementwise_max(amax16, __builtin_bit_cast(u16x2, pk & 0x7FFF7FFFu));
      }
    }
    amax = __uint_as_float((u32)(amax16.x > amax16.y ? amax16.x : amax16.y) << 16);
  } else if constexpr (DT::is_bf16) {
    // tail step: same rule, per-lane reciprocals
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      const float x0 = __uint_as_float(raw[j / 2] << 16), x1 = __uint_as_float(raw[j / 2] & 0xFFFF0000u);
      const float t0 = smooth_bf16(x0, s32[j], y32[j]), t1 = smooth_bf16(x1, s32[j + 1], y32[j + 1]);
      amax = fmaxf(amax, fmaxf(fabsf(t0), fabsf(t1)));
      xb[j / 2] = pack_bf16x2(t0, t1);
    }
    amax = __uint_as_float((u32)BF16::from_f32(amax) << 16);
  } else {
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      float x0, x1;
      if constexpr (DT::is_bf16) {
        x0 = __uint_as_float(raw[j / 2] << 16);
        x1 = __uint_as_float(raw[j / 2] & 0xFFFF0000u);
      } else {
        x0 = __uint_as_float(raw[j]);
        x1 = __uint_as_float(raw[j + 1]);
      }
      const float q0 = div_rn(x0, s32[j], y32[j]);
      const float q1 = div_rn(x1, s32[j + 1], y32[j + 1]);
      if constexpr (DT::is_bf16) {
        const u32 pk = pack_bf16x2(q0, q1);
        xb[j / 2] = pk;
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(pk << 16)), fabsf(__uint_as_float(pk & 0xFFFF0000u))));
      } else {
        xb[j] = __float_as_uint(q0);
        xb[j + 1] = __float_as_uint(q1);
        amax = fmaxf(amax, fmaxf(fabsf(q0), fabsf(q1)));
      }
    }
  }
  st.amax = amax;
}

// Second half of a step: activation codes (block or per-tensor scale) and the step's share of
// down = X^ L1 on the matrix cores.
template <class DT, int FMT, bool NIB, int RC>
__device__ __forceinline__ void act_finish(const ActParams& p, const ActLane& L, int k0, v4f* acc,
                                           const StepState<DT, RC>& st) {
  typedef typename DT::T T;
  constexpr int NB = RC / 16;
  const int k = k0 + 32 * L.g;
  const T* __restrict__ l1t = reinterpret_cast<const T*>(p.l1t);
  const u32* xb = st.xb;
  const auto& bw = st.bw;
  const float amax = st.amax;
  auto val = [&](int j) -> float {
    if constexpr (DT::is_bf16)
      return (j & 1) ? __uint_as_float(xb[j / 2] & 0xFFFF0000u) : __uint_as_float(xb[j / 2] << 16);
    else
      return __uint_as_float(xb[j]);
  };
  // INT codes of the step's 32 values: clamp(rint(RN_f32(z / s_x))). The fast product
  // t = RN(z * RN(1/s_x)) (|t| <= qmax + 1, so 8 ulps < 2^-14) rounds to the same integer
  // unless it lies within 2^-14 of a half-integer; the largest distance to the nearest integer
  // is kept, and when any lane of the wave saw one that close (or s_x has no stored
  // reciprocal) the whole step takes the correctly rounded quotients. s_x = 0 (an all-zero
  // tensor) gives code 0. The quotient is clamped to [-qmax, qmax] first (qmax is an integer,
  // so this commutes with the rounding) and rounded by adding 1.5 * 2^23: the sum's low
  // mantissa bits then hold the code, ties to even, in two's complement (tb[j]).
  auto int_codes = [&](u32* tb) {
    constexpr float SH = 0x1.8p23f;
    const bool int_fast = L.ysx != 0.f;
    float worst = 0.f;
    if (int_fast) {
#pragma unroll
      for (int j = 0; j < 32; j++) {
        const float d = __builtin_amdgcn_fmed3f(val(j) * L.ysx, -L.qmax, L.qmax);
        const float t = d + SH;
        worst = fmaxf(worst, fabsf(d - (t - SH)));
        tb[j] = __float_as_uint(t);
      }
    }
    if (__any(!int_fast || worst >= 0.5f - 0x1p-14f)) {
#pragma unroll
      for (int j = 0; j < 32; j++) {
        const float d = L.sx == 0.f ? 0.f : __builtin_amdgcn_fmed3f(div_rn(val(j), L.sx, L.ysx), -L.qmax, L.qmax);
        tb[j] = __float_as_uint(d + SH);
      }
    }
  };
  if (L.do_codes && L.b < p.B) {
    if constexpr (FMT == SVDQ_FMT_MX) {
      // two-level scaling quantises z = RN(X^ g_x): the block maximum of |z| is RN(amax g_x)
      // (a positive scale and the rounding are monotone)
      const bool scaled = L.gx != 1.f;
      const int e = mx_exponent(scaled ? amax * L.gx : amax);
      const float sc = pow2f(e);
      u32 w4[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        if (DT::is_bf16 && !scaled) {
          w4[q] = fp4_pack8_bf16(&xb[4 * q], sc);
        } else {
          float v[8];
#pragma unroll
          for (int h = 0; h < 8; h++) v[h] = val(8 * q + h) * L.gx;
          w4[q] = fp4_pack8(v, sc);
        }
      }
      const int64_t co = p.codes_tiled ? (((int64_t)(L.b >> 4) * (p.Kp >> 7) + (k >> 7)) << 10) + ((L.b & 15) << 6) + ((k & 127) >> 1)
                                       : (int64_t)L.b * p.ldc + k / 2;
      *reinterpret_cast<uint4*>(p.codes + co) = uint4{w4[0], w4[1], w4[2], w4[3]};
      const int64_t si = p.mxs_tiled ? mx_scale_tiled_index(L.b, k / 32, p.Kp / 128) : (int64_t)L.b * p.lds + k / 32;
      p.mxs[si] = (uint8_t)(e + 127);
    } else if constexpr (NIB) {
      u32 c[32];
      int_codes(c);
      u32 ws[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        u32 r = 0;
#pragma unroll
        for (int h = 0; h < 8; h++) r |= (c[8 * q + h] & 0xFu) << (4 * h);
        ws[q] = r;
      }
      *reinterpret_cast<uint4*>(p.codes + (int64_t)L.b * p.ldc + k / 2) = uint4{ws[0], ws[1], ws[2], ws[3]};
    } else {
      u32 c[32];
      int_codes(c);
      u32 ws[8];
#pragma unroll
      for (int q = 0; q < 8; q++) {
        u32 r = 0;
#pragma unroll
        for (int h = 0; h < 4; h++) r |= (c[4 * q + h] & 0xFFu) << (8 * h);
        ws[q] = r;
      }
      uint4* dst = reinterpret_cast<uint4*>(p.codes + (int64_t)L.b * p.ldc + k);
      dst[0] = uint4{ws[0], ws[1], ws[2], ws[3]};
      dst[1] = uint4{ws[4], ws[5], ws[6], ws[7]};
    }
  }
  if (L.nbl > 0) {
    if constexpr (DT::is_bf16) {
      v8bf av[4];
#pragma unroll
      for (int s = 0; s < 4; s++)
        av[s] = __builtin_bit_cast(v8bf, v4i{(int)xb[4 * s], (int)xb[4 * s + 1], (int)xb[4 * s + 2], (int)xb[4 * s + 3]});
#pragma unroll
      for (int n = 0; n < NB; n++)
        if (n < L.nbl) {
#pragma unroll
          for (int s = 0; s < 4; s++)
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s], __builtin_bit_cast(v8bf, bw[n][s]), acc[n], 0, 0, 0);
        }
    } else {
      // f32: 16x16x4 MFMAs; K-slice c of the tile holds k0 + 32 g + 4 c + e for e < 4
#pragma unroll
      for (int n = 0; n < NB; n++)
        if (n < L.nbl) {
          const float* tile = reinterpret_cast<const float*>(l1t) +
                              ((int64_t)(L.rbase / 16 + n) * (p.Kp / 128) + k0 / 128) * 2048 + L.lane * 4;
#pragma unroll
          for (int c = 0; c < 8; c++) {
            const float4 l4 = *reinterpret_cast<const float4*>(tile + c * 256);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; e++)
              acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(xb[4 * c + e]), lv[e], acc[n], 0, 0, 0);
          }
        }
    }
  }
}


// One 128-wide K step of one wave (see the kernel comment). FULL bf16 steps take their x and
// reciprocals from `in` (loaded by the caller one step ahead); other steps load their own.
template <class DT, int FMT, bool NIB, bool FULL, int RC>
__device__ __forceinline__ void act_step(const ActParams& p, const typename DT::T* __restrict__ xrow, const ActLane& L,
                                         int k0, v4f* acc, const FullIn<RC>& in, const v4i (&bwc)[RC / 16][4]) {
  StepState<DT, RC> st;
  act_smooth<DT, FMT, NIB, FULL, RC>(p, xrow, L, k0, in, bwc, st);
  act_finish<DT, FMT, NIB, RC>(p, L, k0, acc, st);
}

// LR: the block has low-rank columns (rank > 0; then every block has at least one 16-wide tile).
// ONE: K chunks of at most one step per wave (decode and small batches), so no wave prefetches.
template <class DT, int FMT, bool NIB, int RC, bool LR, bool ONE>
__global__ __launch_bounds__(512) void k_act_quant(ActParams p) {
  typedef typename DT::T T;
  constexpr int NW = ACT_WAVES;
  __shared__ float red[NW][16][RC];
  ActLane L;
  L.lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  L.i = L.lane & 15;
  L.g = L.lane >> 4;
  const int row0 = blockIdx.x * 16;
  L.b = row0 + L.i;
  const int bl = L.b < p.B ? L.b : p.B - 1;
  const int kbeg = blockIdx.y * p.k_chunk_len;
  const int kend = kbeg + p.k_chunk_len < p.Kp ? kbeg + p.k_chunk_len : p.Kp;
  L.rbase = blockIdx.z * RC;
  L.nbl = p.rp > L.rbase ? ((p.rp - L.rbase) >= RC ? RC / 16 : (p.rp - L.rbase) / 16) : 0;
  // The rank chunks of one (rows, K range) all smooth it; the codes are split between them by
  // waves: waves 0-3 code in chunk 0 and waves 4-7 in chunk 1 (both in the only chunk when
  // there is one), so a SIMD (waves s and s + 4) codes at most one step per round.
  static_assert(NW == 8, "the code split below pairs waves s and s + 4 of a SIMD");
  L.do_codes = p.codes != nullptr && (int)((wave / 4) % gridDim.z) == (int)blockIdx.z;
  const T* __restrict__ xrow = reinterpret_cast<const T*>(p.x) + (int64_t)bl * p.ldx;
  // full bf16 steps load x by quads (load_full), from the block's first row; rows past B read
  // row B - 1 like the lane's own row does
  const T* __restrict__ xblk = reinterpret_cast<const T*>(p.x) + (int64_t)row0 * p.ldx;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int r = 4 * (L.i >> 2) + q;
    L.xoff[q] = (row0 + r < p.B ? r : p.B - 1 - row0) * (int)p.ldx + 32 * L.g + 8 * (L.i & 3);
  }

  // the first full bf16 step's x, scales and reciprocals are requested before the per-tensor
  // maximum is read, so that the two memory round trips overlap
  // (the quad loads' 32-bit offsets need 17 row strides to fit in an int)
  const int kfull = (p.x_vec_ok && p.ldx <= (int64_t)(INT32_MAX / 17)) ? p.M : 0;
  int k0 = kbeg + 128 * wave;
  FullIn<RC> cur;
  const bool full0 = DT::is_bf16 && k0 < kend && k0 + 128 <= kfull;
  if constexpr (DT::is_bf16)
    if (full0) load_full<RC, LR>(p, xblk, L, k0, cur);

  L.sx = 0.f;
  L.ysx = 0.f;
  L.qmax = 0.f;
  L.gx = (FMT == SVDQ_FMT_MX && p.gscale) ? p.gscale[0] : 1.f;
  if constexpr (FMT == SVDQ_FMT_INT) {
    // each wave reduces the partial maxima on its own (an exact max, so all waves agree), eight
    // loads per lane issued together per 512 partials (one memory round trip instead of one
    // per 64); indices past the last partial re-read it, which leaves the maximum unchanged
    float a = 0.f;
    for (int q0 = 0; q0 < p.n_amax; q0 += 512) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int q = q0 + 64 * u + L.lane;
        v[u] = p.amax_part[q < p.n_amax ? q : p.n_amax - 1];
      }
#pragma unroll
      for (int u = 0; u < 8; u++) a = fmaxf(a, v[u]);
    }
    const float amax = wave_max(a);
    L.qmax = (float)((1 << (p.bits - 1)) - 1);
    L.sx = amax / L.qmax;
    L.ysx = (L.sx >= 0x1p-90f && L.sx <= 0x1p90f) ? 1.0f / L.sx : 0.f;
    if (p.sx_out && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *p.sx_out = L.sx;
  }

  v4f acc[RC / 16];
#pragma unroll
  for (int n = 0; n < RC / 16; n++) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};

  // full steps first (k0 ascending), then the tail and padding; bf16 full steps load the next
  // step's x and reciprocals before computing the current one (a fixed set of loads, so that the
  // compiler's wait for the current step's operands leaves them in flight); a wave's last full
  // step has nothing to prefetch and takes its own copy of the step.
  v4i bwc[RC / 16][4];  // the current full step's L1^T operands when they do not travel ahead
  if constexpr (DT::is_bf16) {
    // ONE: a wave with a single full step takes it without a prefetch. The general loop stays
    // in that instantiation as the other branch (measured faster at decode than without it);
    // other instantiations compile the loop alone.
    const int kn0 = k0 + 128 * NW;
    if (ONE && full0 && !(kn0 < kend && kn0 + 128 <= kfull)) {
      if constexpr (!l1_ahead(RC) && LR) load_l1_all<RC, T>(p, L, k0, bwc);
      act_step<DT, FMT, NIB, true, RC>(p, xrow, L, k0, acc, cur, bwc);
      k0 = kn0;
    } else if (full0) {
      if constexpr (!ONE) {
        // two alternating buffers: the step after next is requested before the wait for the next
        FullIn<RC> nxt;
        // one step: compute from `a` after requesting the next step into `b` (none after the last)
        auto one = [&](FullIn<RC>& a, FullIn<RC>& b) -> bool {
          const int kn = k0 + 128 * NW;
          const bool more = kn < kend && kn + 128 <= kfull;
          if constexpr (!l1_ahead(RC) && LR) load_l1_all<RC, T>(p, L, k0, bwc);  // before the next step's x
          if (!more) {
            act_step<DT, FMT, NIB, true, RC>(p, xrow, L, k0, acc, a, bwc);
            k0 = kn;
            return false;
          }
          load_full<RC, LR>(p, xblk, L, kn, b);
          __builtin_amdgcn_sched_barrier(0);  // the prefetch goes out before any wait on this step's data
          act_step<DT, FMT, NIB, true, RC>(p, xrow, L, k0, acc, a, bwc);
          k0 = kn;
          return true;
        };
        while (one(cur, nxt) && one(nxt, cur)) {
        }
      } else {
        // (the ONE instantiation's fallback keeps the single-buffer loop: measured faster there)
        for (;;) {
          const int kn = k0 + 128 * NW;
          const bool more = kn < kend && kn + 128 <= kfull;
          if constexpr (!l1_ahead(RC) && LR) load_l1_all<RC, T>(p, L, k0, bwc);  // before the next step's x
          if (!more) {  // the wave's last full step: nothing to prefetch
            act_step<DT, FMT, NIB, true, RC>(p, xrow, L, k0, acc, cur, bwc);
            k0 = kn;
            break;
          }
          FullIn<RC> nxt;
          load_full<RC, LR>(p, xblk, L, kn, nxt);
          __builtin_amdgcn_sched_barrier(0);  // the prefetch goes out before any wait on this step's data
          act_step<DT, FMT, NIB, true, RC>(p, xrow, L, k0, acc, cur, bwc);
          k0 = kn;
          cur = nxt;
        }
      }
    }
  } else {
    for (; k0 < kend && k0 + 128 <= kfull; k0 += 128 * NW) act_step<DT, FMT, NIB, true, RC>(p, xrow, L, k0, acc, cur, bwc);
  }
  for (; k0 < kend; k0 += 128 * NW) act_step<DT, FMT, NIB, false, RC>(p, xrow, L, k0, acc, cur, bwc);

  if (L.nbl > 0) {
    // fixed-order sum of the waves' partial down-projections
#pragma unroll
    for (int n = 0; n < RC / 16; n++)
      if (n < L.nbl)
#pragma unroll
        for (int v = 0; v < 4; v++) red[wave][4 * L.g + v][16 * n + L.i] = acc[n][v];
    __syncthreads();
    const int ncols = L.nbl * 16;
    for (int idx = threadIdx.x; idx < 16 * ncols; idx += 64 * NW) {
      const int r = idx / ncols, c = idx - r * ncols;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) s += red[w][r][c];
      const int bb = row0 + r;
      if (bb < p.B) {
        if (p.k_chunks == 1)
          reinterpret_cast<T*>(p.down)[(int64_t)bb * p.rp + L.rbase + c] = DT::from_f32(s);
        else
          p.down_part[(int64_t)blockIdx.y * p.B * p.rp + part_index(p.B, bb, L.rbase + c)] = s;
      }
    }
  }
}

// recip[m] = RN(1 / scale[m]) (IEEE division), or 0 outside [2^-90, 2^90].
__global__ void k_reciprocals(const float* __restrict__ scale, int M, float* __restrict__ recip) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m < M) {
    const float s = scale[m];
    recip[m] = (s >= 0x1p-90f && s <= 0x1p90f) ? 1.0f / s : 0.f;
  }
}


}  // namespace dev

// ------------------------------------------------------------------------- launchers
using namespace dev;

static int grid_for(int64_t n, int cap) {
  int64_t g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

hipError_t launch_smooth(const void* x, int64_t B, int64_t M, int64_t sxb, int64_t sxm, const void* w, int64_t N,
                         int64_t swm, int64_t swn, const float* scale, int dtype, void* xs, int64_t ldxs, void* ws,
                         int64_t ldws, hipStream_t stream) {
  if (x && xs) {
    if (dtype == SVDQ_F32)
      k_smooth_x<F32><<<grid_for(B * M, 4096), 256, 0, stream>>>((const float*)x, B, M, sxb, sxm, scale, (float*)xs, ldxs);
    else
      k_smooth_x<BF16><<<grid_for(B * M, 4096), 256, 0, stream>>>((const uint16_t*)x, B, M, sxb, sxm, scale,
                                                                 (uint16_t*)xs, ldxs);
  }
  if (w && ws) {
    if (dtype == SVDQ_F32)
      k_smooth_w<F32><<<grid_for(M * N, 4096), 256, 0, stream>>>((const float*)w, M, N, swm, swn, scale, (float*)ws, ldws);
    else
      k_smooth_w<BF16><<<grid_for(M * N, 4096), 256, 0, stream>>>((const uint16_t*)w, M, N, swm, swn, scale,
                                                                 (uint16_t*)ws, ldws);
  }
  return hipGetLastError();
}

hipError_t launch_amax_smoothed(const void* x, int B, int M, int64_t ldx, const float* scale, const float* recip,
                                int dtype, float* part, int col_blocks, int row_blocks, hipStream_t stream) {
  const dim3 grid(col_blocks, row_blocks);
  const int rpb = (B + row_blocks - 1) / row_blocks;
  const int esz = dtype == SVDQ_F32 ? 4 : 2;
  const int vec_ok = (((uintptr_t)x & 15) == 0) && ((ldx * esz) % 16 == 0);
  if (dtype == SVDQ_F32)
    k_amax_cols<F32><<<grid, 256, 0, stream>>>((const float*)x, B, M, ldx, scale, recip, rpb, vec_ok, part);
  else
    k_amax_cols<BF16><<<grid, 256, 0, stream>>>((const uint16_t*)x, B, M, ldx, scale, recip, rpb, vec_ok, part);
  return hipGetLastError();
}

hipError_t launch_amax(const void* z, int64_t rows, int64_t cols, int64_t szr, int64_t szc, const float* scale,
                       int dtype, float* part, int nparts, hipStream_t stream) {
  if (dtype == SVDQ_F32) {
    if (scale)
      k_amax_part<F32, true><<<nparts, 256, 0, stream>>>((const float*)z, rows, cols, szr, szc, scale, part);
    else
      k_amax_part<F32, false><<<nparts, 256, 0, stream>>>((const float*)z, rows, cols, szr, szc, scale, part);
  } else {
    if (scale)
      k_amax_part<BF16, true><<<nparts, 256, 0, stream>>>((const uint16_t*)z, rows, cols, szr, szc, scale, part);
    else
      k_amax_part<BF16, false><<<nparts, 256, 0, stream>>>((const uint16_t*)z, rows, cols, szr, szc, scale, part);
  }
  return hipGetLastError();
}

hipError_t launch_fake_quant(const void* z, int64_t rows, int64_t cols, int64_t szr, int64_t szc, int dtype, int bits,
                             const float* part, int nparts, void* out, int64_t ldo, float* s_out, hipStream_t stream) {
  const int grid = grid_for(rows * cols, 2048);
  if (dtype == SVDQ_F32)
    k_fake_quant<F32><<<grid, 256, 0, stream>>>((const float*)z, rows, cols, szr, szc, bits, part, nparts, (float*)out,
                                                ldo, s_out);
  else
    k_fake_quant<BF16><<<grid, 256, 0, stream>>>((const uint16_t*)z, rows, cols, szr, szc, bits, part, nparts,
                                                 (uint16_t*)out, ldo, s_out);
  return hipGetLastError();
}

hipError_t launch_reciprocals(const float* scale, int M, float* recip, hipStream_t stream) {
  k_reciprocals<<<(M + 255) / 256, 256, 0, stream>>>(scale, M, recip);
  return hipGetLastError();
}

hipError_t launch_act_quant(const ActParams& p, int fmt, int dtype, int row_blocks, int r_chunks, int rchunk,
                            hipStream_t stream) {
  const dim3 grid(row_blocks, p.k_chunks, r_chunks);
  const int threads = 64 * ACT_WAVES;
  const bool nib = fmt == SVDQ_FMT_MX || p.bits <= 4;
  // at most one K step per wave (K chunks of up to 128 x waves): the bf16 form without prefetch
  const bool one = dtype == SVDQ_BF16 && p.k_chunk_len <= 128 * ACT_WAVES;
#define SVDQ_ACT(DT, FMT, NIB)                                                    \
  do {                                                                             \
    if (p.rp == 0 && one)                                                          \
      k_act_quant<DT, FMT, NIB, 16, false, true><<<grid, threads, 0, stream>>>(p);  \
    else if (p.rp == 0)                                                            \
      k_act_quant<DT, FMT, NIB, 16, false, false><<<grid, threads, 0, stream>>>(p); \
    else if (rchunk == 16 && one)                                                  \
      k_act_quant<DT, FMT, NIB, 16, true, true><<<grid, threads, 0, stream>>>(p);   \
    else if (rchunk == 16)                                                         \
      k_act_quant<DT, FMT, NIB, 16, true, false><<<grid, threads, 0, stream>>>(p);  \
    else if (rchunk == 32)                                                         \
      k_act_quant<DT, FMT, NIB, 32, true, false><<<grid, threads, 0, stream>>>(p);  \
    else                                                                           \
      k_act_quant<DT, FMT, NIB, 64, true, false><<<grid, threads, 0, stream>>>(p);  \
  } while (0)
  if (!p.recip || (rchunk != 16 && rchunk != 32 && rchunk != 64)) return hipErrorInvalidValue;
  if (dtype == SVDQ_BF16) {
    if (fmt == SVDQ_FMT_MX)
      SVDQ_ACT(BF16, SVDQ_FMT_MX, true);
    else if (nib)
      SVDQ_ACT(BF16, SVDQ_FMT_INT, true);
    else
      SVDQ_ACT(BF16, SVDQ_FMT_INT, false);
  } else {
    if (fmt == SVDQ_FMT_MX)
      SVDQ_ACT(F32, SVDQ_FMT_MX, true);
    else if (nib)
      SVDQ_ACT(F32, SVDQ_FMT_INT, true);
    else
      SVDQ_ACT(F32, SVDQ_FMT_INT, false);
  }
#undef SVDQ_ACT
  return hipGetLastError();
}


}  // namespace svdq
