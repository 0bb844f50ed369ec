// Residual GEMM for MXFP4 at decode-sized batch (B <= 64) on gfx950 (step (c) of the operator):
//   Y = D( Q(X^) Q(R) + down L2 ),
// bound by streaming the packed residual R once from HBM.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 3; "flashinfer.gemm.svdquant_linear" (residual GEMM with the low-rank up-projection in
// its epilogue); msModelSlim SVDQuant guide step 2 (MXFP4 per block).
//
// Structure: v_mfma_scale_f32_16x16x128_f8f6f4 with the (up to 64) batch rows as the M side in
// 16-row tiles. A block owns 32 output columns (two 16-column tiles); its eight waves (two per
// SIMD; four waves for batches above 32 rows) split K evenly. Each lane loads its 32-code K
// block of a weight column straight into registers in the MFMA B layout (every weight byte is
// used once, so there is no LDS staging); the prepared codes are tiled so that a 16-column
// step is one contiguous 1 KB load, and so are the activation codes of a 16-row tile. Eight K steps per batch so that many requests are in
// flight; at 16 rows and K = 8192 each wave's whole share is one batch. Each wave adds its share of
// the up-projection down L2 (16 rank columns per wave, bf16 MFMAs) to its partial tile; those
// operands are requested ahead of the residual codes and multiplied while the codes are still
// in flight. The partial tiles are summed in LDS in a fixed order, and one wave rounds and
// stores.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

constexpr int DEC_COLS = 32;   // output columns per block

// MT: 16-row tiles of the batch; DEC_WAVES: waves per block, each taking 1/DEC_WAVES of K
// (eight, two per SIMD, while the registers allow; four with four row tiles). DT: the io
// dtype (x, down, L2, bias and Y): bf16 takes the up-projection on bf16 MFMAs, f32 on f32
// MFMAs (16x16x4) with no rounding of its operands.
template <class DT, int MT, int DEC_WAVES>
__global__ __launch_bounds__(64 * DEC_WAVES) void k_gemm_decode_mx(GemmParams p) {
  typedef typename DT::T T;
  // up-projection operands of one lane: four consecutive rank entries as stored
  typedef typename std::conditional<DT::is_bf16, v4s, v4f>::type U4;
  constexpr int DEC_BATCH = MT >= 2 ? 4 : 8;  // K steps per load batch
  __shared__ float red[DEC_WAVES][MT][2][64][4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * DEC_COLS;
  const int nst = p.kq;  // 128-code K steps
  const int s0 = (wave * nst) / DEC_WAVES, s1 = ((wave + 1) * nst) / DEC_WAVES;

  // weight columns of the two tiles and activation rows of the MT tiles for this lane
  const uint8_t* wsrc[2];
  const uint8_t* wssrc[2];
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    int col = n0 + 16 * tt + i;
    col = col < p.npad ? col : p.npad - 1;
    wsrc[tt] = p.wcodes + mx_code_tile_offset(col, p.kq) + g * 16;  // + 1024 per K step
    wssrc[tt] = p.wscales + mx_scale_tiled_index(col, 0, p.kq);
  }
  // activation codes: 16-row x 128-code tiles (one contiguous 1 KB per MFMA operand, + 1 KB per
  // K step) when the activation kernel wrote them so, else row-major (+ 64 bytes per K step)
  const uint8_t* asrc[MT];
  const uint8_t* assrc[MT];
  const int astep = p.acodes_tiled ? 1024 : 64;
#pragma unroll
  for (int m = 0; m < MT; m++) {
    int row = 16 * m + i;
    row = row < p.B ? row : p.B - 1;
    asrc[m] = p.acodes + (p.acodes_tiled ? ((int64_t)(row >> 4) * p.kq << 10) + (row & 15) * 64 : (int64_t)row * p.lda) + g * 16;
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

  // ---- up-projection operands. Wave w owns rank columns [16 w + UPW j, +16) for j = 0, 1, ...
  // (lane (i, g) holds down[row i][4 g .. 4 g + 3] and L2^T[col i][same]; bf16: one 16x16x16
  // MFMA per tile, f32: four 16x16x4 MFMAs, the e-th taking entries 4 g + e of the lanes).
  // down is either the finished [B][rp] matrix or the sum, in chunk order, of the f32 split-K
  // partials (rounded once to bf16 for bf16 io). Round j = 0 is loaded before the residual codes, so its
  // requests travel together with them and its MFMAs run while the codes are still in flight.
  constexpr int UPW = 16 * DEC_WAVES;
  constexpr int PF = MT >= 4 ? 2 : 8 / MT;  // split-K partials prefetched per round (the rest are summed after)
  const T* l2t = reinterpret_cast<const T*>(p.l2t);
  int urow[MT], ucol[2];
#pragma unroll
  for (int m = 0; m < MT; m++) urow[m] = 16 * m + i < p.B ? 16 * m + i : p.B - 1;
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    const int col = n0 + 16 * tt + i;
    ucol[tt] = col < p.npad ? col : p.npad - 1;
  }
  struct UpOps {
    U4 b[2];
    v4f part[MT][PF];  // split-K partials (down_chunks > 1)
    U4 d[MT];          // finished down entries (down_chunks <= 1)
  };
  auto up_load = [&](UpOps& u, int kk) {
#pragma unroll
    for (int tt = 0; tt < 2; tt++) u.b[tt] = *reinterpret_cast<const U4*>(l2t + (int64_t)ucol[tt] * p.rp + kk);
    if (p.down_chunks <= 1) {
#pragma unroll
      for (int m = 0; m < MT; m++)
        u.d[m] = *reinterpret_cast<const U4*>(reinterpret_cast<const T*>(p.down) + (int64_t)urow[m] * p.rp + kk);
    } else {
      const int64_t stride = (int64_t)p.B * p.rp;
#pragma unroll
      for (int m = 0; m < MT; m++)
#pragma unroll
        for (int c = 0; c < PF; c++)
          if (c < p.down_chunks)
            u.part[m][c] = *reinterpret_cast<const v4f*>(p.down_part + c * stride + part_index(p.B, urow[m], kk));
    }
  };
  auto up_mma = [&](const UpOps& u, int kk) {
#pragma unroll
    for (int m = 0; m < MT; m++) {
      U4 a;
      if (p.down_chunks <= 1) {
        a = u.d[m];
      } else {
        v4f sum = u.part[m][0];
#pragma unroll
        for (int c = 1; c < PF; c++)
          if (c < p.down_chunks) sum += u.part[m][c];
        const int64_t stride = (int64_t)p.B * p.rp;
        for (int c = PF; c < p.down_chunks; c++)
          sum += *reinterpret_cast<const v4f*>(p.down_part + c * stride + part_index(p.B, urow[m], kk));
        if constexpr (DT::is_bf16) {
          const u32 lo = pack_bf16x2(sum[0], sum[1]), hi = pack_bf16x2(sum[2], sum[3]);
          a = __builtin_bit_cast(v4s, v2u{lo, hi});
        } else {
          a = sum;
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; tt++) {
        if constexpr (DT::is_bf16) {
          acc[m][tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, u.b[tt], acc[m][tt], 0, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++) acc[m][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], u.b[tt][e], acc[m][tt], 0, 0, 0);
        }
      }
    }
  };
  const int kk0 = 16 * wave + 4 * g;  // this lane's first rank column of round 0
  const bool up0 = 16 * wave < p.rp;
  UpOps u0;
  if (up0) up_load(u0, kk0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- residual product over this wave's K range, DEC_BATCH steps per load batch
  struct Batch {
    v4i wv[DEC_BATCH][2], av[DEC_BATCH][MT];
    u32 wsc[DEC_BATCH][2], asc[DEC_BATCH][MT];
  };
  auto batch_load = [&](Batch& bt, int s) {
#pragma unroll
    for (int u = 0; u < DEC_BATCH; u++) {
#pragma unroll
      for (int tt = 0; tt < 2; tt++) {
        bt.wv[u][tt] = *reinterpret_cast<const v4i*>(wsrc[tt] + (int64_t)(s + u) * 1024);
        bt.wsc[u][tt] = *reinterpret_cast<const u32*>(wssrc[tt] + (int64_t)(s + u) * 256);
      }
#pragma unroll
      for (int m = 0; m < MT; m++) {
        bt.av[u][m] = *reinterpret_cast<const v4i*>(asrc[m] + (int64_t)(s + u) * astep);
        bt.asc[u][m] = *reinterpret_cast<const u32*>(assrc[m] + (int64_t)(s + u) * 256);
      }
    }
  };
  // The first batch is peeled: its loads go out before the up-projection's operands are summed
  // and multiplied (inside a loop the compiler would hoist that sum, and its wait, above them).
  int s = s0;
  if (s + DEC_BATCH <= s1) {
    Batch bt;
    batch_load(bt, s);
    __builtin_amdgcn_sched_barrier(0);
    if (up0) up_mma(u0, kk0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < DEC_BATCH; u++) step(bt.wv[u], bt.wsc[u], bt.av[u], bt.asc[u]);
    s += DEC_BATCH;
  } else if (up0) {
    up_mma(u0, kk0);  // no full batch
  }
  for (; s + DEC_BATCH <= s1; s += DEC_BATCH) {
    Batch bt;
    batch_load(bt, s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < DEC_BATCH; u++) step(bt.wv[u], bt.wsc[u], bt.av[u], bt.asc[u]);
  }
  for (; s < s1; s++) {
    v4i wv[2], av[MT];
    u32 wsc[2], asc[MT];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      wv[tt] = *reinterpret_cast<const v4i*>(wsrc[tt] + (int64_t)s * 1024);
      wsc[tt] = *reinterpret_cast<const u32*>(wssrc[tt] + (int64_t)s * 256);
    }
#pragma unroll
    for (int m = 0; m < MT; m++) {
      av[m] = *reinterpret_cast<const v4i*>(asrc[m] + (int64_t)s * astep);
      asc[m] = *reinterpret_cast<const u32*>(assrc[m] + (int64_t)s * 256);
    }
    step(wv, wsc, av, asc);
  }
  // later up-projection rounds (rank above 16 x waves)
  for (int kk = kk0 + UPW; kk - 4 * g < p.rp; kk += UPW) {
    UpOps u;
    up_load(u, kk);
    up_mma(u, kk);
  }

  // fixed-order sum of the waves' partial tiles
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
      {
        float sum = red[0][m][tt][lane][v];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; w++) sum += red[w][m][tt][lane][v];
        acc[m][tt][v] = sum;
      }

  const float al = p.alpha ? p.alpha[0] : 1.f;  // two-level MX scaling (applied before the bias)
  T* y = reinterpret_cast<T*>(p.y);
#pragma unroll
  for (int m = 0; m < MT; m++)
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const int col = n0 + 16 * tt + i;
      const float bz = bias_at<DT>(p.bias, col, p.N);
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int row = 16 * m + 4 * g + v;
        if (row < p.B) __builtin_nontemporal_store(DT::from_f32(acc[m][tt][v] * al + bz), y + (int64_t)row * p.ldy + col);
      }
    }
}

}  // namespace dev

using namespace dev;

template <class DT>
static hipError_t launch_decode_t(const GemmParams& p, hipStream_t stream) {
  const int grid = (p.N + DEC_COLS - 1) / DEC_COLS;
  if (p.B <= 16)
    return launch_gemm_kernel(k_gemm_decode_mx<DT, 1, 8>, dim3(grid), dim3(512), 0, stream, p);
  else if (p.B <= 32)
    return launch_gemm_kernel(k_gemm_decode_mx<DT, 2, 8>, dim3(grid), dim3(512), 0, stream, p);
  else
    return launch_gemm_kernel(k_gemm_decode_mx<DT, 4, 4>, dim3(grid), dim3(256), 0, stream, p);
}

hipError_t launch_gemm_mx_decode(const GemmParams& p, int dtype, hipStream_t stream) {
  if (p.B > 64) return hipErrorNotSupported;
  return dtype == SVDQ_BF16 ? launch_decode_t<BF16>(p, stream) : launch_decode_t<F32>(p, stream);
}

}  // namespace svdq
