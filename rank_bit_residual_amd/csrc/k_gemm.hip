// Step (c) of the operator on gfx950 matrix cores:
//   Y = D( Q(X^) Q(R) + down L2 )
// with the residual product on block-scaled FP4 MFMAs (MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4,
// one E8M0 byte per lane scaling that lane's 32-element K block) or int8 MFMAs (per-tensor
// INT, exact int32 accumulation, dequantised by s_x * s_R in the epilogue). The up-projection
// down L2 runs on bf16 (or fp32) MFMAs into the same fp32 accumulators.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 3 (Y = (X^ L1) L2 + Q(X^) Q(R)); "flashinfer.gemm.svdquant_linear" (the residual GEMM
// with the low-rank up-projection fused into its epilogue is prior art for this split).
//
// It serves the shapes the specialised kernels decline: operand arrays past 2 GiB, which they
// address through buffer resources with 32-bit offsets (this kernel uses 64-bit addresses).
//
// Tiling: a 128x128 output tile per 256-thread block (2x2 waves of 64x64, each 2x2 MFMA
// tiles of 32x32). K advances in stages of 128 bytes per row (256 FP4 / INT4 codes or 128
// int8 codes), double-buffered in LDS; rows are stored as eight 16-byte chunks at position
// chunk ^ (row & 7) so the 16-byte operand reads of 8 consecutive rows hit distinct banks.
#include "device_common.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

constexpr int BM = 128, BN = 128, SB = 128;  // tile rows, tile cols, stage bytes per row

struct GemmSmem {
  uint8_t a[2][BM * SB];
  uint8_t b[2][BN * SB];
  u64 as[2][BM];
  u64 bs[2][BN];
};

__device__ inline int swz(int row, int chunk) { return row * SB + ((chunk ^ (row & 7)) << 4); }

template <class DT, int FMT, bool NIB>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  typedef typename DT::T T;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  GemmSmem& sm = *reinterpret_cast<GemmSmem*>(smem_raw);
  constexpr bool MX = FMT == SVDQ_FMT_MX;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;

  // global -> LDS assignment: 4 chunks of A and 4 of B per thread per stage
  const int ld_row = t >> 3, ld_ch = t & 7;
  const uint8_t* a_src[4];
  const uint8_t* b_src[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    int ra = m0 + ld_row + 32 * j;
    ra = ra < p.B ? ra : p.B - 1;
    a_src[j] = p.acodes + (int64_t)ra * p.lda + ld_ch * 16;
    const int n = n0 + ld_row + 32 * j;
    // MX weight codes are tiled (1 KB per 16 columns x 128 codes; a 256-code stage spans two
    // tiles 1 KB apart); INT codes are K-contiguous rows
    b_src[j] = MX ? p.wcodes + mx_code_tile_offset(n, p.kq) + (ld_ch & 3) * 16 + (ld_ch >> 2) * 1024
                  : p.wcodes + (int64_t)n * p.ldw + ld_ch * 16;
  }
  // scale bytes of one row for a 256-code stage: 4-block groups 2st and 2st+1 (tiled layout)
  const uint8_t* s_src = nullptr;
  if (MX) {
    if (t < BM) {
      int ra = m0 + t;
      ra = ra < p.B ? ra : p.B - 1;
      s_src = p.ascales + mx_scale_tiled_index(ra, 0, p.kq);
    } else {
      s_src = p.wscales + mx_scale_tiled_index(n0 + t - BM, 0, p.kq);
    }
  }

  uint4 ra_[4], rb_[4];
  u64 rs_ = 0;
  auto gload = [&](int st) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      ra_[j] = *reinterpret_cast<const uint4*>(a_src[j] + st * SB);
      rb_[j] = *reinterpret_cast<const uint4*>(b_src[j] + (int64_t)st * (MX ? 2048 : SB));
    }
    if (MX)
      rs_ = (u64) * reinterpret_cast<const u32*>(s_src + (int64_t)(2 * st) * 256) |
            ((u64) * reinterpret_cast<const u32*>(s_src + (int64_t)(2 * st + 1) * 256) << 32);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      *reinterpret_cast<uint4*>(&sm.a[buf][swz(ld_row + 32 * j, ld_ch)]) = ra_[j];
      *reinterpret_cast<uint4*>(&sm.b[buf][swz(ld_row + 32 * j, ld_ch)]) = rb_[j];
    }
    if (MX) {
      if (t < BM)
        sm.as[buf][t] = rs_;
      else
        sm.bs[buf][t - BM] = rs_;
    }
  };

  typedef typename std::conditional<MX, v16f, v16i>::type Acc;
  Acc acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int nt = 0; nt < 2; nt++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[mt][nt][v] = 0;

  const int arow[2] = {64 * wm + l32, 64 * wm + 32 + l32};
  const int bcol[2] = {64 * wn + l32, 64 * wn + 32 + l32};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int st = 0; st < p.kstages; st++) {
    const int buf = st & 1;
    if (st + 1 < p.kstages) gload(st + 1);
    if constexpr (MX) {
      u64 sa[2], sb[2];
#pragma unroll
      for (int q = 0; q < 2; q++) {
        sa[q] = sm.as[buf][arow[q]];
        sb[q] = sm.bs[buf][bcol[q]];
      }
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const int ch = 2 * ks + g;  // this lane's 32-element K block within the stage
        v8i av[2], bv[2];
        int sca[2], scb[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          const v4i a4 = *reinterpret_cast<const v4i*>(&sm.a[buf][swz(arow[q], ch)]);
          const v4i b4 = *reinterpret_cast<const v4i*>(&sm.b[buf][swz(bcol[q], ch)]);
          av[q] = v8i{a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
          bv[q] = v8i{b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
          sca[q] = (int)(u32)(sa[q] >> (8 * ch));
          scb[q] = (int)(u32)(sb[q] >> (8 * ch));
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < 2; nt++)
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[mt], bv[nt], acc[mt][nt], 4, 4, 0,
                                                                          sca[mt], 0, scb[nt]);
      }
    } else if constexpr (NIB) {
#pragma unroll
      for (int ks = 0; ks < 8; ks++) {  // 32 codes (one 16-byte chunk) per K step; lane half g takes 8 bytes
        v4i av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          const uint2 a2 = *reinterpret_cast<const uint2*>(&sm.a[buf][swz(arow[q], ks) + 8 * g]);
          const uint2 b2 = *reinterpret_cast<const uint2*>(&sm.b[buf][swz(bcol[q], ks) + 8 * g]);
          u32 lo0, hi0, lo1, hi1;
          unpack_nibbles(a2.x, lo0, hi0);
          unpack_nibbles(a2.y, lo1, hi1);
          av[q] = v4i{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
          unpack_nibbles(b2.x, lo0, hi0);
          unpack_nibbles(b2.y, lo1, hi1);
          bv[q] = v4i{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < 2; nt++)
            acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {  // 32 int8 codes per K step; lane half g takes chunk 2ks+g
        v4i av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          av[q] = *reinterpret_cast<const v4i*>(&sm.a[buf][swz(arow[q], 2 * ks + g)]);
          bv[q] = *reinterpret_cast<const v4i*>(&sm.b[buf][swz(bcol[q], 2 * ks + g)]);
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < 2; nt++)
            acc[mt][nt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
      }
    }
    if (st + 1 < p.kstages) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: dequantise, add the up-projection, round and store
  v16f f[2][2];
  if constexpr (MX) {
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++) f[mt][nt] = acc[mt][nt];
  } else {
    const float scl = p.sx[0] * p.sr[0];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++)
#pragma unroll
        for (int v = 0; v < 16; v++) f[mt][nt][v] = (float)acc[mt][nt][v] * scl;
  }
  if (p.rp > 0) {
    const T* l2t = reinterpret_cast<const T*>(p.l2t);
    int drow[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int r = m0 + arow[mt];
      drow[mt] = r < p.B ? r : p.B - 1;
    }
    if constexpr (DT::is_bf16) {
      for (int kk = 0; kk < p.rp; kk += 16) {
        v8bf av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          av[q] = down8_bf16(p.down, p.down_part, p.down_chunks, p.B, p.rp, drow[q], kk + 8 * g);
          bv[q] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(l2t + (int64_t)(n0 + bcol[q]) * p.rp + kk + 8 * g));
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < 2; nt++)
            f[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], bv[nt], f[mt][nt], 0, 0, 0);
      }
    } else {
      for (int kk = 0; kk < p.rp; kk += 2) {
        float av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          av[q] = down1_f32(p.down, p.down_part, p.down_chunks, p.B, p.rp, drow[q], kk + g);
          bv[q] = l2t[(int64_t)(n0 + bcol[q]) * p.rp + kk + g];
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < 2; nt++)
            f[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt], bv[nt], f[mt][nt], 0, 0, 0);
      }
    }
  }
  if (p.alpha) {  // two-level MX scaling: alpha * (residual + down L2 / alpha)
    const float al = p.alpha[0];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++)
#pragma unroll
        for (int v = 0; v < 16; v++) f[mt][nt][v] *= al;
  }
  T* y = reinterpret_cast<T*>(p.y);
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
      const int col = n0 + bcol[nt];
      const float bz = bias_at<DT>(p.bias, col, p.N);
#pragma unroll
      for (int v = 0; v < 16; v++) f[mt][nt][v] += bz;
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int row = m0 + 64 * wm + 32 * mt + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row < p.B) y[(int64_t)row * p.ldy + col] = DT::from_f32(f[mt][nt][v]);
      }
    }
  }
}

}  // namespace dev

using namespace dev;

template <class DT, int FMT, bool NIB>
static hipError_t launch_gemm_t(const GemmParams& p, hipStream_t stream) {
  const dim3 grid((p.N + BN - 1) / BN, (p.B + BM - 1) / BM);
  const size_t smem = sizeof(GemmSmem);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<DT, FMT, NIB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    configured = true;
  }
  return launch_gemm_kernel(k_gemm<DT, FMT, NIB>, grid, dim3(256), smem, stream, p);
}

hipError_t launch_gemm(const GemmParams& p, int fmt, int bits, int dtype, hipStream_t stream) {
  const bool nib = fmt == SVDQ_FMT_MX || bits <= 4;
  if (dtype == SVDQ_BF16) {
    if (fmt == SVDQ_FMT_MX) return launch_gemm_t<BF16, SVDQ_FMT_MX, true>(p, stream);
    if (nib) return launch_gemm_t<BF16, SVDQ_FMT_INT, true>(p, stream);
    return launch_gemm_t<BF16, SVDQ_FMT_INT, false>(p, stream);
  }
  if (fmt == SVDQ_FMT_MX) return launch_gemm_t<F32, SVDQ_FMT_MX, true>(p, stream);
  if (nib) return launch_gemm_t<F32, SVDQ_FMT_INT, true>(p, stream);
  return launch_gemm_t<F32, SVDQ_FMT_INT, false>(p, stream);
}

}  // namespace svdq
