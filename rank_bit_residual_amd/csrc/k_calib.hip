// Smoothing-scale calibration on the device, the step before the operator's path:
//   s[m] = max_b |x[b,m]|^alpha / max_n |W[m,n]|^(1-alpha),   s[m] = 1 where a maximum is 0,
// the power and the quotient in binary64, rounded once to binary32.
//
// Pages: msModelSlim SVDQuant configuration guide, step 2 (iter_smooth alpha, the migration
// strength; 0.25 in its diffusion example), which prints no formula: the closed form above is
// this library's reading, a balance of the two channel maxima. "SVDQuant Smoothing, Low-rank
// and Residual Quantization", "Formula and conventions" item 1 is how the scale is applied.
//
// k_calib_colmax: block (cb, rb) covers columns [64 cb, 64 cb + 64) and a range of rows of x.
// Thread t reads 8 consecutive columns (one 16-byte load for bf16, two for f32) of rows
// t/8, t/8 + 32, ... (eight rows' loads in flight at a time), keeping max |x| per column; the 32 row lanes of a column are combined in
// LDS and the block writes part[rb][m]. All maxima are exact.
// k_calib_finish: one wave per channel m takes the maximum over part[*][m] and over |W[m, :]|
// (16-byte loads along the row), then lane 0 forms s[m].
#include "device_common.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

template <class DT>
__global__ __launch_bounds__(256) void k_calib_colmax(const typename DT::T* __restrict__ x, int B, int M, int64_t ldx,
                                                      int rows_per_block, bool vec_ok, float* __restrict__ part) {
  typedef typename DT::T T;
  constexpr int E = 8;  // columns per thread
  __shared__ float red[32][64 + 1];
  const int t = threadIdx.x, c8 = t & 7, r = t >> 3;
  const int m0 = blockIdx.x * 64 + c8 * E;
  const int b0 = blockIdx.y * rows_per_block;
  const int b1 = b0 + rows_per_block < B ? b0 + rows_per_block : B;
  float mx[E];
#pragma unroll
  for (int e = 0; e < E; e++) mx[e] = 0.f;
  const bool full = vec_ok && m0 + E <= M;
  // U rows per thread and pass, all requested before any is used; rows past the range
  // repeat the last one (harmless for a maximum)
  constexpr int U = 8;
  for (int b = b0 + r; b < b1; b += 32 * U) {
    if (full) {
      uint4 v[U][DT::is_bf16 ? 1 : 2];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int bb = b + 32 * u < b1 ? b + 32 * u : b1 - 1;
        const uint4* row = reinterpret_cast<const uint4*>(x + (int64_t)bb * ldx + m0);
        v[u][0] = row[0];
        if constexpr (!DT::is_bf16) v[u][1] = row[1];
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        if constexpr (DT::is_bf16) {
          const u32 w[4] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w};
#pragma unroll
          for (int q = 0; q < 4; q++) {
            mx[2 * q] = fmaxf(mx[2 * q], fabsf(__uint_as_float(w[q] << 16)));
            mx[2 * q + 1] = fmaxf(mx[2 * q + 1], fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
          }
        } else {
          const u32 w[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w, v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
#pragma unroll
          for (int e = 0; e < E; e++) mx[e] = fmaxf(mx[e], fabsf(__uint_as_float(w[e])));
        }
      }
    } else {
      for (int u = 0; u < U && b + 32 * u < b1; u++) {
        const T* row = x + (int64_t)(b + 32 * u) * ldx + m0;
#pragma unroll
        for (int e = 0; e < E; e++)
          if (m0 + e < M) mx[e] = fmaxf(mx[e], fabsf(DT::to_f32(row[e])));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; e++) red[r][c8 * E + e] = mx[e];
  __syncthreads();
  if (t < 64) {
    float a = red[0][t];
#pragma unroll
    for (int q = 1; q < 32; q++) a = fmaxf(a, red[q][t]);
    const int m = blockIdx.x * 64 + t;
    if (m < M) part[(int64_t)blockIdx.y * M + m] = a;
  }
}

template <class DT>
__global__ __launch_bounds__(256) void k_calib_finish(const float* __restrict__ part, int parts, int M,
                                                      const typename DT::T* __restrict__ w, int N, int64_t ldw,
                                                      bool vec_ok, double alpha, float* __restrict__ scale) {
  typedef typename DT::T T;
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole waves: m is uniform within a wave
  float ax = 0.f;
  for (int q = lane; q < parts; q += 64) ax = fmaxf(ax, part[(int64_t)q * M + m]);
  ax = wave_max(ax);
  const T* row = w + (int64_t)m * ldw;
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte load
  float aw = 0.f;
  int n = 0;
  if (vec_ok) {
    // four 16-byte loads per lane in flight per pass
    for (; n + 4 * 64 * E <= N; n += 4 * 64 * E) {
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; j++) v[j] = *reinterpret_cast<const uint4*>(row + n + (64 * j + lane) * E);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const u32 u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
          if constexpr (DT::is_bf16) {
            aw = fmaxf(aw, fabsf(__uint_as_float(u[q] << 16)));
            aw = fmaxf(aw, fabsf(__uint_as_float(u[q] & 0xFFFF0000u)));
          } else {
            aw = fmaxf(aw, fabsf(__uint_as_float(u[q])));
          }
        }
      }
    }
    for (; n + 64 * E <= N; n += 64 * E) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + n + lane * E);
      const u32 u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        if constexpr (DT::is_bf16) {
          aw = fmaxf(aw, fabsf(__uint_as_float(u[q] << 16)));
          aw = fmaxf(aw, fabsf(__uint_as_float(u[q] & 0xFFFF0000u)));
        } else {
          aw = fmaxf(aw, fabsf(__uint_as_float(u[q])));
        }
      }
    }
  }
  for (int j = n + lane; j < N; j += 64) aw = fmaxf(aw, fabsf(DT::to_f32(row[j])));
  aw = wave_max(aw);
  if (lane == 0) {
    float s = 1.f;
    if (ax > 0.f && aw > 0.f) s = (float)(pow((double)ax, alpha) / pow((double)aw, 1.0 - alpha));
    scale[m] = s;
  }
}

}  // namespace dev

using namespace dev;

int calib_parts(int64_t B, int64_t M) {
  const int64_t col_blocks = (M + 63) / 64;
  int64_t parts = col_blocks >= 256 ? 1 : (256 + col_blocks - 1) / col_blocks;
  const int64_t row_groups = (B + 31) / 32;  // at least 32 rows per block
  if (parts > row_groups) parts = row_groups;
  return (int)(parts < 1 ? 1 : parts);
}

hipError_t launch_calibrate(const void* x, int B, int M, int64_t ldx, const void* w, int N, int64_t ldw, int dtype,
                            double alpha, float* part, float* scale, hipStream_t stream) {
  const int parts = calib_parts(B, M);
  const int rows_per_block = (B + parts - 1) / parts;
  const int esize = dtype == SVDQ_BF16 ? 2 : 4;
  const bool xvec = ((uintptr_t)x % 16 == 0) && (ldx * esize) % 16 == 0;
  const bool wvec = ((uintptr_t)w % 16 == 0) && (ldw * esize) % 16 == 0;
  const dim3 g1((M + 63) / 64, parts), g2((M + 3) / 4);
  if (dtype == SVDQ_BF16) {
    k_calib_colmax<BF16><<<g1, 256, 0, stream>>>((const uint16_t*)x, B, M, ldx, rows_per_block, xvec, part);
    k_calib_finish<BF16><<<g2, 256, 0, stream>>>(part, parts, M, (const uint16_t*)w, N, ldw, wvec, alpha, scale);
  } else {
    k_calib_colmax<F32><<<g1, 256, 0, stream>>>((const float*)x, B, M, ldx, rows_per_block, xvec, part);
    k_calib_finish<F32><<<g2, 256, 0, stream>>>(part, parts, M, (const float*)w, N, ldw, wvec, alpha, scale);
  }
  return hipGetLastError();
}

}  // namespace svdq
