// Residual GEMM for MXFP4 at decode-sized batch (B <= 64) on gfx950 (step (c) of the operator):
//   Y = D( Q(X^) Q(R) + down L2 ),
// bound by streaming the packed residual R once from HBM.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 3; "flashinfer.gemm.svdquant_linear" (residual GEMM with the low-rank up-projection in
// its epilogue); msModelSlim SVDQuant guide step 2 (MXFP4 per block).
//
// Structure: v_mfma_scale_f32_16x16x128_f8f6f4 with the (up to 64) batch rows as the M side in
// 16-row tiles. A 256-thread block owns 32 output columns (two 16-column tiles); its four waves
// split K into quarters. Each lane loads its 32-code K block of a weight column straight into
// registers in the MFMA B layout (every weight byte is used once, so there is no LDS staging),
// eight K steps per batch so that many requests are in flight. Each wave adds its share of
// the up-projection down L2 (bf16 MFMAs) to its partial tile; the four partial tiles are summed
// in LDS in a fixed order, and one wave rounds and stores.
#include "device_common.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

constexpr int DEC_COLS = 32;   // output columns per block
constexpr int DEC_BATCH = 8;   // K steps per load batch

template <int MT>
__global__ __launch_bounds__(256) void k_gemm_decode_mx(GemmParams p) {
  typedef BF16::T T;
  __shared__ float red[4][MT][2][64][4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * DEC_COLS;
  const int nst = p.kq;  // 128-code K steps
  const int s0 = (wave * nst) >> 2, s1 = ((wave + 1) * nst) >> 2;

  // weight columns of the two tiles and activation rows of the MT tiles for this lane
  const uint8_t* wsrc[2];
  const uint8_t* wssrc[2];
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    int col = n0 + 16 * tt + i;
    col = col < p.npad ? col : p.npad - 1;
    wsrc[tt] = p.wcodes + (int64_t)col * p.ldw + g * 16;
    wssrc[tt] = p.wscales + mx_scale_tiled_index(col, 0, p.kq);
  }
  const uint8_t* asrc[MT];
  const uint8_t* assrc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) {
    int row = 16 * m + i;
    row = row < p.B ? row : p.B - 1;
    asrc[m] = p.acodes + (int64_t)row * p.lda + g * 16;
    assrc[m] = p.ascales + mx_scale_tiled_index(row, 0, p.kq);
  }

  v4f acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; m++)
#pragma unroll
    for (int tt = 0; tt < 2; tt++) acc[m][tt] = v4f{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const v4i* wv, const u32* wsc, const v4i* av, const u32* asc) {
#pragma unroll
    for (int m = 0; m < MT; m++)
#pragma unroll
      for (int tt = 0; tt < 2; tt++)
        acc[m][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            v8i{av[m][0], av[m][1], av[m][2], av[m][3], 0, 0, 0, 0},
            v8i{wv[tt][0], wv[tt][1], wv[tt][2], wv[tt][3], 0, 0, 0, 0}, acc[m][tt], 4, 4, 0,
            (int)(asc[m] >> (8 * g)), 0, (int)(wsc[tt] >> (8 * g)));
  };

  int s = s0;
  for (; s + DEC_BATCH <= s1; s += DEC_BATCH) {
    v4i wv[DEC_BATCH][2], av[DEC_BATCH][MT];
    u32 wsc[DEC_BATCH][2], asc[DEC_BATCH][MT];
#pragma unroll
    for (int u = 0; u < DEC_BATCH; u++) {
#pragma unroll
      for (int tt = 0; tt < 2; tt++) {
        wv[u][tt] = *reinterpret_cast<const v4i*>(wsrc[tt] + (int64_t)(s + u) * 64);
        wsc[u][tt] = *reinterpret_cast<const u32*>(wssrc[tt] + (int64_t)(s + u) * 256);
      }
#pragma unroll
      for (int m = 0; m < MT; m++) {
        av[u][m] = *reinterpret_cast<const v4i*>(asrc[m] + (int64_t)(s + u) * 64);
        asc[u][m] = *reinterpret_cast<const u32*>(assrc[m] + (int64_t)(s + u) * 256);
      }
    }
#pragma unroll
    for (int u = 0; u < DEC_BATCH; u++) step(wv[u], wsc[u], av[u], asc[u]);
  }
  for (; s < s1; s++) {
    v4i wv[2], av[MT];
    u32 wsc[2], asc[MT];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      wv[tt] = *reinterpret_cast<const v4i*>(wsrc[tt] + (int64_t)s * 64);
      wsc[tt] = *reinterpret_cast<const u32*>(wssrc[tt] + (int64_t)s * 256);
    }
#pragma unroll
    for (int m = 0; m < MT; m++) {
      av[m] = *reinterpret_cast<const v4i*>(asrc[m] + (int64_t)s * 64);
      asc[m] = *reinterpret_cast<const u32*>(assrc[m] + (int64_t)s * 256);
    }
    step(wv, wsc, av, asc);
  }

  // this wave's share of the up-projection, acc += down[rows, kk..kk+32) . L2^T[cols, kk..kk+32)^T
  // for kk = 32 w, 32 w + 128, ... (16x16x32 bf16 MFMAs), before the partial tiles are summed
  if (p.rp > 0) {
    const T* l2t = reinterpret_cast<const T*>(p.l2t);
    for (int kk = 32 * wave; kk < p.rp; kk += 128) {
      v8bf bv[2];
#pragma unroll
      for (int tt = 0; tt < 2; tt++) {
        int col = n0 + 16 * tt + i;
        col = col < p.npad ? col : p.npad - 1;
        bv[tt] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(l2t + (int64_t)col * p.rp + kk + 8 * g));
      }
#pragma unroll
      for (int m = 0; m < MT; m++) {
        int row = 16 * m + i;
        row = row < p.B ? row : p.B - 1;
        const v8bf av = down8_bf16(p.down, p.down_part, p.down_chunks, p.B, p.rp, row, kk + 8 * g);
#pragma unroll
        for (int tt = 0; tt < 2; tt++) acc[m][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[tt], acc[m][tt], 0, 0, 0);
      }
    }
  }

  // fixed-order sum of the four waves' partial tiles
#pragma unroll
  for (int m = 0; m < MT; m++)
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int v = 0; v < 4; v++) red[wave][m][tt][lane][v] = acc[m][tt][v];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MT; m++)
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int v = 0; v < 4; v++)
        acc[m][tt][v] = ((red[0][m][tt][lane][v] + red[1][m][tt][lane][v]) + red[2][m][tt][lane][v]) +
                        red[3][m][tt][lane][v];

  T* y = reinterpret_cast<T*>(p.y);
#pragma unroll
  for (int m = 0; m < MT; m++)
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const int col = n0 + 16 * tt + i;
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int row = 16 * m + 4 * g + v;
        if (row < p.B) y[(int64_t)row * p.ldy + col] = BF16::from_f32(acc[m][tt][v]);
      }
    }
}

}  // namespace dev

using namespace dev;

hipError_t launch_gemm_mx_decode(const GemmParams& p, int dtype, hipStream_t stream) {
  if (dtype != SVDQ_BF16 || p.B > 64) return hipErrorNotSupported;
  const int grid = (p.N + DEC_COLS - 1) / DEC_COLS;
  if (p.B <= 16)
    k_gemm_decode_mx<1><<<grid, 256, 0, stream>>>(p);
  else if (p.B <= 32)
    k_gemm_decode_mx<2><<<grid, 256, 0, stream>>>(p);
  else
    k_gemm_decode_mx<4><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace svdq
