// Activation-side kernels of libsvdq for gfx950:
//   * k_smooth      — smooth_inputs, elementwise (x / scale, scale * W);
//   * k_amax_part   — per-block maxima of |z| or |x / scale| (per-tensor INT pre-pass);
//   * k_fake_quant  — per-tensor INT fake quantisation (dequantised values);
//   * k_act_quant   — step (a)+(b) of the operator: X^ = D(x / scale), its INT or MXFP4
//                     codes, and the low-rank down-projection X^ L1 on the matrix cores;
//   * k_down_reduce — sums split-K partials of the down-projection in a fixed order.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization" ("Formula and
// conventions" items 1 and 3: smoothing divides x by scale; the low-rank branch takes the
// unquantised smoothed activations; per-tensor INT with ties to even) and the msModelSlim
// SVDQuant guide, step 2 (MXFP4 per-block minmax activations).
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
    xs[b * ldxs + m] = DT::from_f32(DT::to_f32(x[b * sxb + m * sxm]) / scale[m]);
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
  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < M) {
    for (int r = r0; r < r1; r++) {
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
    if (c0 + q < M) {
      const float y = recip ? recip[c0 + q] : 0.f;
      a = fmaxf(a, DT::to_f32(DT::from_f32(div_rn(cm[q], scale[c0 + q], y))));
    }
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
constexpr int ACT_WAVES = 8;
constexpr int ACT_RCHUNK = 64;

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

// 8 consecutive entries of a per-channel float array (scale or reciprocal); `pad` past M.
__device__ inline void load8(const float* __restrict__ a, int k, int M, float pad, float* v) {
  if (k + 8 <= M) {
    const float4 u = *reinterpret_cast<const float4*>(a + k), w = *reinterpret_cast<const float4*>(a + k + 4);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w; v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = (k + j < M) ? a[k + j] : pad;
  }
}

template <class DT, int FMT, bool NIB>
__global__ __launch_bounds__(512) void k_act_quant(ActParams p) {
  typedef typename DT::T T;
  constexpr int NW = ACT_WAVES;
  __shared__ float red[NW][16][ACT_RCHUNK];
  __shared__ float sh[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int b = row0 + i;
  const int bl = b < p.B ? b : p.B - 1;
  const int kbeg = blockIdx.y * p.k_chunk_len;
  const int kend = kbeg + p.k_chunk_len < p.Kp ? kbeg + p.k_chunk_len : p.Kp;
  const int rbase = blockIdx.z * ACT_RCHUNK;
  const int nbl = p.rp > rbase ? ((p.rp - rbase) >= ACT_RCHUNK ? ACT_RCHUNK / 16 : (p.rp - rbase) / 16) : 0;
  const bool do_codes = blockIdx.z == 0 && p.codes != nullptr;
  const T* __restrict__ xrow = reinterpret_cast<const T*>(p.x) + (int64_t)bl * p.ldx;
  const T* __restrict__ l1t = reinterpret_cast<const T*>(p.l1t);

  float sx = 0.f, ysx = 0.f, qmax = 0.f;
  if constexpr (FMT == SVDQ_FMT_INT) {
    // the 512-thread block reduces the per-block maxima in two 256-thread halves
    float a = 0.f;
    for (int q = threadIdx.x; q < p.n_amax; q += 512) a = fmaxf(a, p.amax_part[q]);
    a = wave_max(a);
    __shared__ float shw[NW];
    if (lane == 0) shw[wave] = a;
    __syncthreads();
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < NW; q++) amax = fmaxf(amax, shw[q]);
    qmax = (float)((1 << (p.bits - 1)) - 1);
    sx = amax / qmax;
    ysx = (sx >= 0x1p-90f && sx <= 0x1p90f) ? 1.0f / sx : 0.f;
    if (p.sx_out && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *p.sx_out = sx;
  }
  (void)sh;

  v4f acc[ACT_RCHUNK / 16];
#pragma unroll
  for (int n = 0; n < ACT_RCHUNK / 16; n++) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg + 128 * wave; k0 < kend; k0 += 128 * NW) {
    const int k = k0 + 32 * g;
    constexpr int RW = DT::is_bf16 ? 16 : 32;
    u32 raw[RW];
    load_row32<DT>(xrow, k, p.M, p.x_vec_ok, raw);
    // X^ = D(x / scale) in chunks of 8; xb: X^ as stored (bf16 pairs or f32 bits)
    u32 xb[RW];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float s8[8], y8[8];
      load8(p.scale, k + 8 * c, p.M, 1.f, s8);
      if (p.recip)
        load8(p.recip, k + 8 * c, p.M, 1.f, y8);
      else
#pragma unroll
        for (int j = 0; j < 8; j++) y8[j] = 0.f;
#pragma unroll
      for (int h = 0; h < 4; h++) {
        const int j = 8 * c + 2 * h;
        if constexpr (DT::is_bf16) {
          const u32 w = raw[j / 2];
          const float q0 = div_rn(__uint_as_float(w << 16), s8[2 * h], y8[2 * h]);
          const float q1 = div_rn(__uint_as_float(w & 0xFFFF0000u), s8[2 * h + 1], y8[2 * h + 1]);
          typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
          typedef float f2 __attribute__((ext_vector_type(2)));
          const u32 pk = __builtin_bit_cast(u32, __builtin_convertvector(f2{q0, q1}, bf2));
          xb[j / 2] = pk;
          amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(pk << 16)), fabsf(__uint_as_float(pk & 0xFFFF0000u))));
        } else {
          const float q0 = div_rn(__uint_as_float(raw[j]), s8[2 * h], y8[2 * h]);
          const float q1 = div_rn(__uint_as_float(raw[j + 1]), s8[2 * h + 1], y8[2 * h + 1]);
          xb[j] = __float_as_uint(q0);
          xb[j + 1] = __float_as_uint(q1);
          amax = fmaxf(amax, fmaxf(fabsf(q0), fabsf(q1)));
        }
      }
    }
    auto val = [&](int j) -> float {
      if constexpr (DT::is_bf16)
        return (j & 1) ? __uint_as_float(xb[j / 2] & 0xFFFF0000u) : __uint_as_float(xb[j / 2] << 16);
      else
        return __uint_as_float(xb[j]);
    };
    if (do_codes && b < p.B) {
      if constexpr (FMT == SVDQ_FMT_MX) {
        const int e = mx_exponent(amax);
        const float sc = pow2f(e);
        u32 w4[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          float v[8];
#pragma unroll
          for (int h = 0; h < 8; h++) v[h] = val(8 * q + h);
          w4[q] = fp4_pack8(v, sc);
        }
        *reinterpret_cast<uint4*>(p.codes + (int64_t)b * p.ldc + k / 2) = uint4{w4[0], w4[1], w4[2], w4[3]};
        const int64_t si = p.mxs_tiled ? mx_scale_tiled_index(b, k / 32, p.Kp / 128) : (int64_t)b * p.lds + k / 32;
        p.mxs[si] = (uint8_t)(e + 127);
      } else if constexpr (NIB) {
        u32 ws[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          u32 r = 0;
#pragma unroll
          for (int h = 0; h < 8; h++) {
            const float z = val(8 * q + h);
            const int c = sx == 0.f ? 0 : (int)fminf(fmaxf(__builtin_rintf(div_rn(z, sx, ysx)), -qmax), qmax);
            r |= (u32)(c & 0xF) << (4 * h);
          }
          ws[q] = r;
        }
        *reinterpret_cast<uint4*>(p.codes + (int64_t)b * p.ldc + k / 2) = uint4{ws[0], ws[1], ws[2], ws[3]};
      } else {
        u32 ws[8];
#pragma unroll
        for (int q = 0; q < 8; q++) {
          u32 r = 0;
#pragma unroll
          for (int h = 0; h < 4; h++) {
            const float z = val(4 * q + h);
            const int c = sx == 0.f ? 0 : (int)fminf(fmaxf(__builtin_rintf(div_rn(z, sx, ysx)), -qmax), qmax);
            r |= (u32)(c & 0xFF) << (8 * h);
          }
          ws[q] = r;
        }
        uint4* dst = reinterpret_cast<uint4*>(p.codes + (int64_t)b * p.ldc + k);
        dst[0] = uint4{ws[0], ws[1], ws[2], ws[3]};
        dst[1] = uint4{ws[4], ws[5], ws[6], ws[7]};
      }
    }
    if (nbl > 0) {
      if constexpr (DT::is_bf16) {
        v4i bw[ACT_RCHUNK / 16][4];
#pragma unroll
        for (int n = 0; n < ACT_RCHUNK / 16; n++)
          if (n < nbl) {
            const T* tile = l1t + ((int64_t)(rbase / 16 + n) * (p.Kp / 128) + k0 / 128) * 2048 + lane * 8;
#pragma unroll
            for (int s = 0; s < 4; s++) bw[n][s] = *reinterpret_cast<const v4i*>(tile + s * 512);
          }
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const v8bf av = __builtin_bit_cast(v8bf, v4i{(int)xb[4 * s], (int)xb[4 * s + 1], (int)xb[4 * s + 2], (int)xb[4 * s + 3]});
#pragma unroll
          for (int n = 0; n < ACT_RCHUNK / 16; n++)
            if (n < nbl) acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, bw[n][s]), acc[n], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int n = 0; n < ACT_RCHUNK / 16; n++) {
          if (n < nbl) {
            const float* tile = reinterpret_cast<const float*>(l1t) +
                                ((int64_t)(rbase / 16 + n) * (p.Kp / 128) + k0 / 128) * 2048 + lane * 4;
#pragma unroll
            for (int c = 0; c < 8; c++) {
              const float4 lr = *reinterpret_cast<const float4*>(tile + c * 256);
              const float l4[4] = {lr.x, lr.y, lr.z, lr.w};
#pragma unroll
              for (int e = 0; e < 4; e++)
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(xb[4 * c + e]), l4[e], acc[n], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  if (nbl > 0) {
    // fixed-order sum of the waves' partial down-projections
#pragma unroll
    for (int n = 0; n < ACT_RCHUNK / 16; n++)
      if (n < nbl)
#pragma unroll
        for (int v = 0; v < 4; v++) red[wave][4 * g + v][16 * n + i] = acc[n][v];
    __syncthreads();
    const int ncols = nbl * 16;
    for (int idx = threadIdx.x; idx < 16 * ncols; idx += 64 * NW) {
      const int r = idx / ncols, c = idx - r * ncols;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) s += red[w][r][c];
      const int bb = row0 + r;
      if (bb < p.B) {
        if (p.k_chunks == 1)
          reinterpret_cast<T*>(p.down)[(int64_t)bb * p.rp + rbase + c] = DT::from_f32(s);
        else
          p.down_part[((int64_t)blockIdx.y * p.B + bb) * p.rp + rbase + c] = s;
      }
    }
  }
}

// Fixed-order sum of the split-K partials; the independent loads of a thread are issued
// together so their latencies overlap.
template <class DT>
__global__ void k_down_reduce(const float* __restrict__ part, int k_chunks, int B, int rp,
                              typename DT::T* __restrict__ down) {
  const int n = B * rp;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
    float s = 0.f;
    int c = 0;
    for (; c + 8 <= k_chunks; c += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; q++) v[q] = part[(int64_t)(c + q) * n + idx];
#pragma unroll
      for (int q = 0; q < 8; q++) s += v[q];
    }
    for (; c < k_chunks; c++) s += part[(int64_t)c * n + idx];
    down[idx] = DT::from_f32(s);
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

hipError_t launch_act_quant(const ActParams& p, int fmt, int dtype, int row_blocks, int r_chunks, hipStream_t stream) {
  const dim3 grid(row_blocks, p.k_chunks, r_chunks);
  const int threads = 64 * ACT_WAVES;
  const bool nib = fmt == SVDQ_FMT_MX || p.bits <= 4;
  if (dtype == SVDQ_BF16) {
    if (fmt == SVDQ_FMT_MX)
      k_act_quant<BF16, SVDQ_FMT_MX, true><<<grid, threads, 0, stream>>>(p);
    else if (nib)
      k_act_quant<BF16, SVDQ_FMT_INT, true><<<grid, threads, 0, stream>>>(p);
    else
      k_act_quant<BF16, SVDQ_FMT_INT, false><<<grid, threads, 0, stream>>>(p);
  } else {
    if (fmt == SVDQ_FMT_MX)
      k_act_quant<F32, SVDQ_FMT_MX, true><<<grid, threads, 0, stream>>>(p);
    else if (nib)
      k_act_quant<F32, SVDQ_FMT_INT, true><<<grid, threads, 0, stream>>>(p);
    else
      k_act_quant<F32, SVDQ_FMT_INT, false><<<grid, threads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_down_reduce(const float* part, int k_chunks, int B, int rp, void* down, int dtype,
                              hipStream_t stream) {
  const int grid = grid_for((int64_t)B * rp, 1024);
  if (dtype == SVDQ_F32)
    k_down_reduce<F32><<<grid, 256, 0, stream>>>(part, k_chunks, B, rp, (float*)down);
  else
    k_down_reduce<BF16><<<grid, 256, 0, stream>>>(part, k_chunks, B, rp, (uint16_t*)down);
  return hipGetLastError();
}

}  // namespace svdq
