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

// ------------------------------------------------------------------------- step (a) + (b)
// Block (rb, kc, rc): rows [16 rb, 16 rb + 16), K range [kc * k_chunk_len, ...), low-rank
// columns [128 rc, 128 rc + 128). Four waves walk the K range in 128-wide steps. In a step,
// lane l owns row l % 16 and the whole 32-element block l / 16 of that step: the block max,
// shared exponent and codes stay inside the lane. For the down-projection the lane feeds the
// same 32 values to the matrix cores: 16x16x32 bf16 MFMAs in four K-slices of 8 (the B
// operand lane (n, g) supplies L1^T[n] at the same K offsets, so the K order is consistent).
template <class DT>
__device__ inline void load_row32(const typename DT::T* __restrict__ xrow, int k, int M, bool vec_ok, float* v) {
  if (vec_ok && k + 32 <= M) {
    if constexpr (DT::is_bf16) {
      const uint4* p = reinterpret_cast<const uint4*>(xrow + k);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint4 w = p[q];
        const u32 ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; h++) {
          v[8 * q + 2 * h] = __uint_as_float(ws[h] << 16);
          v[8 * q + 2 * h + 1] = __uint_as_float(ws[h] & 0xFFFF0000u);
        }
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(xrow + k);
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const float4 w = p[q];
        v[4 * q] = w.x;
        v[4 * q + 1] = w.y;
        v[4 * q + 2] = w.z;
        v[4 * q + 3] = w.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; j++) v[j] = (k + j < M) ? DT::to_f32(xrow[k + j]) : 0.f;
  }
}

__device__ inline void load_scale32(const float* __restrict__ scale, int k, int M, float* s) {
  if (k + 32 <= M) {
    const float4* p = reinterpret_cast<const float4*>(scale + k);
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const float4 w = p[q];
      s[4 * q] = w.x;
      s[4 * q + 1] = w.y;
      s[4 * q + 2] = w.z;
      s[4 * q + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; j++) s[j] = (k + j < M) ? scale[k + j] : 1.f;
  }
}

template <class DT, int FMT, bool NIB>
__global__ __launch_bounds__(256) void k_act_quant(ActParams p) {
  typedef typename DT::T T;
  __shared__ float red[4][16][128];
  __shared__ float sh[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int b = row0 + i;
  const int bl = b < p.B ? b : p.B - 1;
  const int kbeg = blockIdx.y * p.k_chunk_len;
  const int kend = kbeg + p.k_chunk_len < p.Kp ? kbeg + p.k_chunk_len : p.Kp;
  const int rbase = blockIdx.z * 128;
  const int nbl = p.rp > rbase ? ((p.rp - rbase) >= 128 ? 8 : (p.rp - rbase) / 16) : 0;
  const bool do_codes = blockIdx.z == 0 && p.codes != nullptr;
  const T* __restrict__ xrow = reinterpret_cast<const T*>(p.x) + (int64_t)bl * p.ldx;
  const T* __restrict__ l1t = reinterpret_cast<const T*>(p.l1t);

  float sx = 0.f, qmax = 0.f;
  if constexpr (FMT == SVDQ_FMT_INT) {
    const float amax = reduce_parts(p.amax_part, p.n_amax, sh);
    qmax = (float)((1 << (p.bits - 1)) - 1);
    sx = amax / qmax;
    if (p.sx_out && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *p.sx_out = sx;
  }

  v4f acc[8];
#pragma unroll
  for (int n = 0; n < 8; n++) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg + 128 * wave; k0 < kend; k0 += 512) {
    const int k = k0 + 32 * g;
    float xh[32];
    {
      float xv[32], sv[32];
      load_row32<DT>(xrow, k, p.M, p.x_vec_ok, xv);
      load_scale32(p.scale, k, p.M, sv);
#pragma unroll
      for (int j = 0; j < 32; j++) xh[j] = smooth_value<DT>(xv[j], sv[j]);
    }
    if (do_codes && b < p.B) {
      if constexpr (FMT == SVDQ_FMT_MX) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) a = fmaxf(a, fabsf(xh[j]));
        const int e = mx_exponent(a);
        const float sc = pow2f(e);
        uint4 w;
        w.x = fp4_pack8(xh, sc);
        w.y = fp4_pack8(xh + 8, sc);
        w.z = fp4_pack8(xh + 16, sc);
        w.w = fp4_pack8(xh + 24, sc);
        *reinterpret_cast<uint4*>(p.codes + (int64_t)b * p.ldc + k / 2) = w;
        const int64_t si = p.mxs_tiled ? mx_scale_tiled_index(b, k / 32, p.Kp / 128) : (int64_t)b * p.lds + k / 32;
        p.mxs[si] = (uint8_t)(e + 127);
      } else if constexpr (NIB) {
        u32 ws[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          u32 r = 0;
#pragma unroll
          for (int h = 0; h < 8; h++) r |= (u32)(int_code(xh[8 * q + h], sx, qmax) & 0xF) << (4 * h);
          ws[q] = r;
        }
        *reinterpret_cast<uint4*>(p.codes + (int64_t)b * p.ldc + k / 2) = uint4{ws[0], ws[1], ws[2], ws[3]};
      } else {
        u32 ws[8];
#pragma unroll
        for (int q = 0; q < 8; q++) {
          u32 r = 0;
#pragma unroll
          for (int h = 0; h < 4; h++) r |= (u32)(int_code(xh[4 * q + h], sx, qmax) & 0xFF) << (8 * h);
          ws[q] = r;
        }
        uint4* dst = reinterpret_cast<uint4*>(p.codes + (int64_t)b * p.ldc + k);
        dst[0] = uint4{ws[0], ws[1], ws[2], ws[3]};
        dst[1] = uint4{ws[4], ws[5], ws[6], ws[7]};
      }
    }
    if (nbl > 0) {
      if constexpr (DT::is_bf16) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
          v4i ai;
#pragma unroll
          for (int h = 0; h < 4; h++)
            ai[h] = (int)((__float_as_uint(xh[8 * s + 2 * h]) >> 16) | (__float_as_uint(xh[8 * s + 2 * h + 1]) & 0xFFFF0000u));
          const v8bf av = __builtin_bit_cast(v8bf, ai);
#pragma unroll
          for (int n = 0; n < 8; n++) {
            if (n < nbl) {
              const T* lr = l1t + (int64_t)(rbase + 16 * n + i) * p.Kp + k + 8 * s;
              const v8bf bv = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(lr));
              acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
            }
          }
        }
      } else {
#pragma unroll
        for (int n = 0; n < 8; n++) {
          if (n < nbl) {
            const float* lr = reinterpret_cast<const float*>(l1t) + (int64_t)(rbase + 16 * n + i) * p.Kp + k;
#pragma unroll
            for (int s = 0; s < 32; s++) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(xh[s], lr[s], acc[n], 0, 0, 0);
          }
        }
      }
    }
  }

  if (nbl > 0) {
    // fixed-order sum of the four waves' partial down-projections
#pragma unroll
    for (int n = 0; n < 8; n++)
      if (n < nbl)
#pragma unroll
        for (int v = 0; v < 4; v++) red[wave][4 * g + v][16 * n + i] = acc[n][v];
    __syncthreads();
    const int ncols = nbl * 16;
    for (int idx = threadIdx.x; idx < 16 * ncols; idx += 256) {
      const int r = idx / ncols, c = idx - r * ncols;
      const float s = ((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c];
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

template <class DT>
__global__ void k_down_reduce(const float* __restrict__ part, int k_chunks, int B, int rp,
                              typename DT::T* __restrict__ down) {
  const int n = B * rp;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int c = 0; c < k_chunks; c++) s += part[(int64_t)c * n + idx];
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
  const bool nib = fmt == SVDQ_FMT_MX || p.bits <= 4;
  if (dtype == SVDQ_BF16) {
    if (fmt == SVDQ_FMT_MX)
      k_act_quant<BF16, SVDQ_FMT_MX, true><<<grid, 256, 0, stream>>>(p);
    else if (nib)
      k_act_quant<BF16, SVDQ_FMT_INT, true><<<grid, 256, 0, stream>>>(p);
    else
      k_act_quant<BF16, SVDQ_FMT_INT, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (fmt == SVDQ_FMT_MX)
      k_act_quant<F32, SVDQ_FMT_MX, true><<<grid, 256, 0, stream>>>(p);
    else if (nib)
      k_act_quant<F32, SVDQ_FMT_INT, true><<<grid, 256, 0, stream>>>(p);
    else
      k_act_quant<F32, SVDQ_FMT_INT, false><<<grid, 256, 0, stream>>>(p);
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
