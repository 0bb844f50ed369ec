// Residual GEMM for MXFP4 at large batch on gfx950 (step (c) of the operator):
//   Y = D( Q(X^) Q(R) + down L2 )
// Q(X^) and Q(R) are E2M1 codes with one E8M0 scale per 32 elements along K; the product runs
// on v_mfma_scale_f32_32x32x64_f8f6f4 (each lane's 32 K-contiguous FP4 values scaled by its own
// E8M0 byte), fp32 accumulation; the up-projection down L2 runs on bf16 MFMAs into the same
// accumulators before the single rounding to the output dtype.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 3; "flashinfer.gemm.svdquant_linear" (residual GEMM with the low-rank up-projection in
// its epilogue: prior art for this split); msModelSlim SVDQuant guide step 2 (MXFP4 per block).
//
// Structure: a BM x BN output tile per 512-thread block (4 x 2 waves, two per SIMD so that one
// wave's LDS and barrier waits overlap the other's MFMAs). K advances in stages of
// 128 codes (64 bytes per row). Stages land in a ring of NS LDS buffers through direct
// global->LDS loads (global_load_lds_dwordx4 / _dword), issued NS-1 stages ahead; each wave
// waits on its own vmcnt for the stage it is about to read, then one s_barrier makes every
// wave's loads of that stage visible and releases the buffer read in the previous iteration.
// LDS rows are 64 bytes (four 16-byte chunks); chunk c of row r sits at c ^ ((r >> 2) & 3), so
// the 16-byte reads of 16 consecutive rows (one LDS cycle of a ds_read_b128) hit distinct banks.
// The prepared weight codes are tiled 16 columns x 128 codes per 1 KB, so each wave-wide load
// of a B stage reads one contiguous kilobyte (the activation codes are row-major: 16 rows x 64
// bytes per load).
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "gemm_pipe.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

template <int BM, int BN>
struct MxCfg {
  static constexpr int NWV = 8, WN = 2, WM = NWV / WN;  // 4 x 2 waves, two per SIMD
  static constexpr int SB = 64;               // bytes per row per stage (128 FP4 codes)
  static constexpr int TM = BM / WM, TN = BN / WN;  // per-wave tile
  static constexpr int MT = TM / 32, NT = TN / 32;
  static constexpr int A_BYTES = BM * SB, B_BYTES = BN * SB;
  static constexpr int A_INSTR = A_BYTES / 1024, B_INSTR = B_BYTES / 1024;  // wave-wide 16-byte DMA loads
  static_assert(A_INSTR % NWV == 0, "tile rows must fill whole wave-wide loads");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tiles are whole 32 x 32 MFMA tiles");
  static constexpr int A_PER_WAVE = A_INSTR / NWV;
  static constexpr int B_PER_WAVE = (B_INSTR + NWV - 1) / NWV;
  static constexpr int SCALE_BYTES = 1024;         // 256 rows x 4 bytes, per operand (padded)
  static constexpr int STAGE = A_BYTES + B_PER_WAVE * NWV * 1024 + 2 * SCALE_BYTES;
  static constexpr int LOADS_PER_STAGE = A_PER_WAVE + B_PER_WAVE + 1;  // per wave (one scale load)
  static constexpr int NS = 4;    // LDS ring depth
  static constexpr int DIST = 2;  // stages in flight ahead of the one being computed
  static constexpr int SMEM = NS * STAGE;
};

__device__ inline int lds_swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

template <class DT, int BM, int BN>
__global__ __launch_bounds__(512) void k_gemm_mx(GemmParams p) {
  typedef MxCfg<BM, BN> C;
  typedef typename DT::T T;
  extern __shared__ __align__(1024) uint8_t smem[];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int l32 = lane & 31, g = lane >> 5;

  // ---- tile order: XCD-aware (blocks i, i+8, ... share an XCD) and grouped by 4 row tiles
  const int tiles_m = (p.B + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int tid = blockIdx.x;
  if ((ntiles & 7) == 0) tid = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int GM = 4;
  const int group = tid / (GM * tiles_n);
  const int gm0 = group * GM;
  const int gsz = (tiles_m - gm0) < GM ? (tiles_m - gm0) : GM;
  const int in_g = tid - group * GM * tiles_n;
  const int tm = gm0 + in_g % gsz, tn = in_g / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- per-lane DMA sources (16-byte chunks) for this wave's share of a stage
  const uint8_t* a_src[C::A_PER_WAVE];
  int a_dst[C::A_PER_WAVE];
#pragma unroll
  for (int j = 0; j < C::A_PER_WAVE; j++) {
    const int u = wave + C::NWV * j;  // instruction index: 16 rows x 64 bytes
    const int q = u * 64 + lane;
    const int row = q >> 2, phys = q & 3;
    const int chunk = phys ^ ((row >> 2) & 3);
    int gr = m0 + row;
    gr = gr < p.B ? gr : p.B - 1;
    a_src[j] = p.acodes + (int64_t)gr * p.lda + chunk * 16;
    a_dst[j] = u * 1024;
  }
  const uint8_t* b_src[C::B_PER_WAVE];
  int b_dst[C::B_PER_WAVE];
#pragma unroll
  for (int j = 0; j < C::B_PER_WAVE; j++) {
    int u = wave + C::NWV * j;
    const bool real = u < C::B_INSTR;
    const int q = (real ? u : 0) * 64 + lane;
    const int row = q >> 2, phys = q & 3;
    const int chunk = phys ^ ((row >> 2) & 3);
    int gr = n0 + row;
    gr = gr < p.npad ? gr : p.npad - 1;
    b_src[j] = p.wcodes + mx_code_tile_offset(gr, p.kq) + chunk * 16;  // tiled: + 1024 per stage
    b_dst[j] = C::A_BYTES + u * 1024;  // u >= B_INSTR lands in the padding after B
  }
  // scales (stage-tiled): waves 0-3 load the 64-row groups 0-3 of the A tile, waves 4-7 those of
  // the B tile, 256 contiguous bytes per stage; groups past the data clamp to the last one
  // (discarded)
  const int sw = wave & 3;
  int ga = (m0 >> 6) + sw;
  ga = ga < p.ascale_groups ? ga : p.ascale_groups - 1;
  const uint8_t* sa_src = p.ascales + ((int64_t)ga * p.kq << 8) + lane * 4;
  int gb = (n0 >> 6) + (64 * sw < BN ? sw : 0);
  gb = gb < (p.npad >> 6) ? gb : (p.npad >> 6) - 1;
  const uint8_t* sb_src = p.wscales + ((int64_t)gb * p.kq << 8) + lane * 4;
  const int s_off_a = C::A_BYTES + C::B_PER_WAVE * C::NWV * 1024;
  const int s_off_b = s_off_a + C::SCALE_BYTES;

  auto issue = [&](int st) {
    uint8_t* base = smem + (st % C::NS) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::A_PER_WAVE; j++)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[j] + st * C::SB), (lds_ptr_t)(base + a_dst[j]), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < C::B_PER_WAVE; j++)
      __builtin_amdgcn_global_load_lds((const void*)(b_src[j] + (int64_t)st * 1024), (lds_ptr_t)(base + b_dst[j]), 16, 0, 0);
    if (wave < 4)
      __builtin_amdgcn_global_load_lds((const void*)(sa_src + st * 256), (lds_ptr_t)(base + s_off_a + sw * 256), 4, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(sb_src + st * 256), (lds_ptr_t)(base + s_off_b + sw * 256), 4, 0, 0);
  };

  v16f acc[C::MT][C::NT];
#pragma unroll
  for (int i = 0; i < C::MT; i++)
#pragma unroll
    for (int j = 0; j < C::NT; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // Operand fragment of one 64-code K slice: A rows and B columns of this wave's tile read
  // from the LDS stage buffer.
  struct Frag {
    v8i a[C::MT], b[C::NT];
  };
  // Scale words of a stage: four E8M0 bytes (one per 32-code block) per row / column.
  struct Scales {
    u32 a[C::MT], b[C::NT];
  };
  auto read_frag = [&](const uint8_t* base, int ks, Frag& f) {
    const int ch = 2 * ks + g;  // this lane's 32-code K block within the stage
#pragma unroll
    for (int i = 0; i < C::MT; i++) {
      const v4i a4 = *reinterpret_cast<const v4i*>(base + lds_swz(wm * C::TM + 32 * i + l32, ch));
      f.a[i] = v8i{a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < C::NT; j++) {
      const v4i b4 = *reinterpret_cast<const v4i*>(base + C::A_BYTES + lds_swz(wn * C::TN + 32 * j + l32, ch));
      f.b[j] = v8i{b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
    }
  };
  auto read_scales = [&](const uint8_t* base, Scales& sc) {
#pragma unroll
    for (int i = 0; i < C::MT; i++)
      sc.a[i] = *reinterpret_cast<const u32*>(base + s_off_a + (wm * C::TM + 32 * i + l32) * 4);
#pragma unroll
    for (int j = 0; j < C::NT; j++)
      sc.b[j] = *reinterpret_cast<const u32*>(base + s_off_b + (wn * C::TN + 32 * j + l32) * 4);
  };
  auto mma = [&](const Frag& f, const Scales& sc, int ks) {
    const int sh = 8 * (2 * ks + g);
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
      for (int j = 0; j < C::NT; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, 0,
                                                                    (int)(sc.a[i] >> sh), 0, (int)(sc.b[j] >> sh));
  };

  // Pipeline: stage s+DIST is issued into the ring at the top of iteration s; slice 1 of stage s
  // is read from LDS while slice 0's MFMAs run; then the wave waits until its own loads of
  // stage s+1 have landed, one barrier publishes every wave's loads of that stage, and stage
  // s+1's scale words and slice-0 operands are read while slice 1's MFMAs of stage s run. No LDS
  // round trip is exposed between stages, and the MFMAs issued before the barrier keep the
  // matrix core busy while the waves meet. The barrier of stage s+1 (in iteration s) is also
  // what makes refilling buffer (s+1+DIST) % NS = (s-1) % NS safe in iteration s+1: every
  // wave's reads of stage s-1 were consumed by MFMAs issued before it (NS = DIST + 2).
  static_assert(C::NS >= C::DIST + 2, "ring too shallow for the prefetch distance");
  constexpr int NR = C::MT + C::NT;  // 16-byte operand reads per slice
  constexpr int NM = C::MT * C::NT;  // MFMAs per slice
  static_assert(NM > NR, "the interleave schedule assumes more MFMAs than operand reads per slice");
  const int nst = p.kstages;

  // ---- up-projection first: acc = down L2 on bf16 32x32x16 MFMAs. Its first 32 rank columns
  // are requested before the first stages' DMA and multiplied while those stages land; the
  // residual product then accumulates on top (one rounding at the end either way).
  const T* l2t = reinterpret_cast<const T*>(p.l2t);
  int drow[C::MT], bcol[C::NT];
#pragma unroll
  for (int i = 0; i < C::MT; i++) {
    const int r = m0 + wm * C::TM + 32 * i + l32;
    drow[i] = r < p.B ? r : p.B - 1;
  }
#pragma unroll
  for (int j = 0; j < C::NT; j++) {
    const int c = n0 + wn * C::TN + 32 * j + l32;
    bcol[j] = c < p.npad ? c : p.npad - 1;
  }
  struct UpOps {
    v8bf a[2][C::MT], b[2][C::NT];
  };
  auto up_load = [&](UpOps& u, int kk) {  // rank columns [kk, kk + 32), rp a multiple of 32
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int i = 0; i < C::MT; i++)
        u.a[h][i] = down8_bf16_pf<2>(p.down, p.down_part, p.down_chunks, p.B, p.rp, drow[i], kk + 16 * h + 8 * g);
#pragma unroll
      for (int j = 0; j < C::NT; j++)
        u.b[h][j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(l2t + (int64_t)bcol[j] * p.rp + kk + 16 * h + 8 * g));
    }
  };
  auto up_mma = [&](const UpOps& u) {
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u.a[h][i], u.b[h][j], acc[i][j], 0, 0, 0);
  };
  UpOps u0;
  if (p.rp > 0) up_load(u0, 0);
#pragma unroll
  for (int s = 0; s < C::DIST; s++)
    if (s < nst) issue(s);
  if (p.rp > 0) {
    up_mma(u0);
    for (int kk = 32; kk < p.rp; kk += 32) {
      UpOps u;
      up_load(u, kk);
      up_mma(u);
    }
  }

  wait_stage<C::LOADS_PER_STAGE, C::DIST + 2>(nst - 1 < C::DIST - 1 ? nst - 1 : C::DIST - 1);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Frag fa, fb, f1;
  Scales sa, sb;
  read_scales(smem, sa);
  read_frag(smem, 0, fa);

  // One stage: cur0/scur hold stage s's slice-0 operands and scales; nxt0/snxt receive stage
  // s+1's unless AHEAD < 0 (the last stage). AHEAD = stages issued after s+1.
  auto stage = [&](int s, Frag& cur0, Scales& scur, Frag& nxt0, Scales& snxt, auto ahead_c) {
    constexpr int AHEAD = decltype(ahead_c)::value;
    const uint8_t* base = smem + (s % C::NS) * C::STAGE;
    read_frag(base, 1, f1);
    mma(cur0, scur, 0);
    // slice 1's reads one per slice-0 MFMA
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int q = 0; q < NR; q++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NR - 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (AHEAD >= 0) {
      wait_vmcnt<C::LOADS_PER_STAGE * AHEAD>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const uint8_t* nb = smem + ((s + 1) % C::NS) * C::STAGE;
      read_scales(nb, snxt);
      read_frag(nb, 0, nxt0);
    }
    mma(f1, scur, 1);
    // the next stage's scale words and slice-0 reads one per slice-1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int q = 0; q < 2 * NR; q++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (q < NM - 1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - 1 > 2 * NR ? NM - 1 - 2 * NR : 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  typedef std::integral_constant<int, C::DIST - 1> Steady;
  typedef std::integral_constant<int, 0> LastButOne;
  typedef std::integral_constant<int, -1> Last;

  // Steady state: every iteration issues stage s + DIST and has DIST - 1 stages in flight after
  // s + 1; unrolled by two so that the slice-0 operands alternate between fa and fb. nst is
  // even (Kp is a multiple of 256) and DIST = 2, so the loop leaves exactly the last two stages.
  static_assert(C::DIST == 2, "the drain below is written for two stages in flight");
  for (int s = 0; s < nst - C::DIST; s += 2) {
    issue(s + C::DIST);
    stage(s, fa, sa, fb, sb, Steady());
    issue(s + 1 + C::DIST);
    stage(s + 1, fb, sb, fa, sa, Steady());
  }
  stage(nst - 2, fa, sa, fb, sb, LastButOne());
  stage(nst - 1, fb, sb, fa, sa, Last());

  // ---- two-level scaling: alpha * (residual + down L2 / alpha), before the bias
  if (p.alpha) {
    const float al = p.alpha[0];
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
      for (int j = 0; j < C::NT; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][j][v] *= al;
  }

  // ---- output bias (one column per lane and 32x32 tile)
  if (p.bias) {
#pragma unroll
    for (int j = 0; j < C::NT; j++) {
      const float bz = bias_at<DT>(p.bias, n0 + wn * C::TN + 32 * j + l32, p.N);
#pragma unroll
      for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[i][j][v] += bz;
    }
  }

  // ---- epilogue: one rounding, staged through the (now idle) LDS ring for 16-byte stores. In a
  // 32x32 tile lane (l32, g) holds column l32 of rows 8q + 4g + e (e = 0..3). Neighbouring lanes
  // swap one value (DPP quad_perm [1,0,3,2]) so that the even lane holds row 8q + 4g + e,
  // columns (l32, l32+1) and the odd lane row 8q + 4g + e + 1 of the same two columns
  // (e = 0, 2): one 4-byte LDS write per pair.
  static_assert(BM * BN * 2 <= C::SMEM, "output tile must fit the LDS ring");
  const bool odd = l32 & 1;
  __syncthreads();
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < C::MT; i++)
#pragma unroll
    for (int j = 0; j < C::NT; j++) {
      const int c = wn * C::TN + 32 * j + (l32 & ~1);
#pragma unroll
      for (int q = 0; q < 4; q++)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float m0v = acc[i][j][4 * q + e], m1v = acc[i][j][4 * q + e + 1];
          const float send = odd ? m0v : m1v;
          const float recv = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
          const u32 w = odd ? pack_bf16x2(recv, m1v) : pack_bf16x2(m0v, recv);
          const int r = wm * C::TM + 32 * i + 8 * q + 4 * g + e + (odd ? 1 : 0);
          *reinterpret_cast<u32*>(tile + r * BN + c) = w;
        }
    }
  __syncthreads();
  T* y = reinterpret_cast<T*>(p.y);
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  const bool vec_ok = (p.ldy % 8 == 0) && (((uintptr_t)p.y & 15) == 0);
  for (int c = t; c < BM * CPR; c += 64 * C::NWV) {
    const int r = c / CPR, cc = c - r * CPR;
    const int row = m0 + r, col = n0 + cc * 8;
    if (row >= p.B || col >= p.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + r * BN + cc * 8);
    T* dst = y + (int64_t)row * p.ldy + col;
    if (vec_ok && col + 8 <= p.N) {
      // streaming store: the output is not read again here, so it should not push the operand
      // stages that other tiles of this XCD still read out of L2
      __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, reinterpret_cast<v4i*>(dst));
    } else {
      const u32 w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 8; q++)
        if (col + q < p.N) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
    }
  }
}

}  // namespace dev

using namespace dev;

template <int BM, int BN>
static hipError_t launch_mx_t(const GemmParams& p, hipStream_t stream) {
  typedef MxCfg<BM, BN> C;
  const int tiles = ((p.B + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mx<BF16, BM, BN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    if (e != hipSuccess) return e;
    configured = true;
  }
  return launch_gemm_kernel(k_gemm_mx<BF16, BM, BN>, dim3(tiles), dim3(64 * C::NWV), C::SMEM, stream, p);
}

// Large-batch MXFP4 path for bf16 inputs; returns hipErrorNotSupported when the shape or dtype
// is not covered, so the caller falls back to the general kernel.
hipError_t launch_gemm_mx_large(const GemmParams& p, int dtype, hipStream_t stream) {
  if (dtype != SVDQ_BF16 || p.B < 256 || p.kstages < 2 || p.kstages % 2) return hipErrorNotSupported;
  // 256 x 256 tiles move the least operand data per flop; 256 x 192 fills the chip better when
  // there are few tiles (e.g. N = 3072 gives 12 column tiles of 256 but 16 of 192).
  const int tiles_m = (p.B + 255) / 256;
  if (p.N % 256 == 0 && tiles_m * (p.N / 256) >= 512) return launch_mx_t<256, 256>(p, stream);
  if (p.N % 192 == 0) return launch_mx_t<256, 192>(p, stream);
  return launch_mx_t<256, 256>(p, stream);
}

}  // namespace svdq
