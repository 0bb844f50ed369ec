// Residual GEMM at large batch on gfx950 (step (c) of the operator), for MXFP4 (k_gemm_mx)
// and for per-tensor INT4 (k_gemm_int_big, the same body on int8 MFMAs; see gemm_big):
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
// The prepared weight codes are tiled 16 columns x 128 codes per 1 KB, and the activation
// kernel writes the MXFP4 activation codes for this kernel in the same 1 KB tiles of 16 rows,
// so each wave-wide load of a stage reads one contiguous kilobyte (INT operands are row-major:
// 16 rows x 64 bytes per load).
#include <atomic>
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

// Eight f32 values as bf16 high parts RN(v) and low parts RN(v - RN(v)).
__device__ inline void split_bf16x8(const float* v, v8bf& hi, v8bf& lo) {
  u32 h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    h[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    const float r0 = v[2 * q] - __uint_as_float(h[q] << 16), r1 = v[2 * q + 1] - __uint_as_float(h[q] & 0xFFFF0000u);
    l[q] = pack_bf16x2(r0, r1);
  }
  hi = __builtin_bit_cast(v8bf, v4i{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
  lo = __builtin_bit_cast(v8bf, v4i{(int)l[0], (int)l[1], (int)l[2], (int)l[3]});
}

// f32 output of a BM x BN tile: staged through the idle LDS ring in CH row chunks (a whole f32
// tile is larger than the ring), each written by the waves whose rows it holds (one 4-byte LDS
// write per value) and stored as 16-byte streaming stores.
template <int BM, int BN, int MT, int NT>
__device__ __forceinline__ void store_f32_tile(const GemmParams& p, const v16f (&acc)[MT][NT], uint8_t* smem, int t,
                                               int wm, int wn, int l32, int g, int m0, int n0) {
  typedef MxCfg<BM, BN> C;
  constexpr int CH = (BM * BN * 4 + C::SMEM - 1) / C::SMEM;
  static_assert(CH == 1 || CH == 2 || CH == 4, "row chunks must split the four wave rows evenly");
  constexpr int CR = BM / CH;  // rows per chunk
  float* tile = reinterpret_cast<float*>(smem);
  float* y = reinterpret_cast<float*>(p.y);
  constexpr int CPR = BN / 4;  // 16-byte chunks per tile row
  const bool vec_ok = (p.ldy % 4 == 0) && (((uintptr_t)p.y & 15) == 0);
#pragma unroll
  for (int ch = 0; ch < CH; ch++) {
    __syncthreads();
    if (wm / (C::WM / CH) == ch) {
#pragma unroll
      for (int i = 0; i < MT; i++)
#pragma unroll
        for (int j = 0; j < NT; j++)
#pragma unroll
          for (int v = 0; v < 16; v++) {
            const int r = wm * C::TM + 32 * i + 8 * (v / 4) + 4 * g + (v % 4) - ch * CR;
            tile[r * BN + wn * C::TN + 32 * j + l32] = acc[i][j][v];
          }
    }
    __syncthreads();
    for (int c = t; c < CR * CPR; c += 64 * C::NWV) {
      const int r = c / CPR, cc = c - r * CPR;
      const int row = m0 + ch * CR + r, col = n0 + cc * 4;
      if (row >= p.B || col >= p.N) continue;
      const float4 v = *reinterpret_cast<const float4*>(tile + r * BN + cc * 4);
      float* dst = y + (int64_t)row * p.ldy + col;
      if (vec_ok && col + 4 <= p.N) {
        __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(dst));
      } else {
        const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; q++)
          if (col + q < p.N) dst[q] = w[q];
      }
    }
  }
}

// One BM x BN tile of the residual GEMM. INTC = false: MXFP4 (FP4 codes with E8M0 scales,
// weight codes tiled 16 columns x 128 codes per 1 KB). INTC = true: per-tensor INT, both
// operands row-major and K-contiguous, no per-block scales, a stage still 64 bytes per row.
// NIB (nibble codes, 128 per stage): each FP4 MFMA's slot becomes two int8 MFMAs on the odd
// and even codes (a nibble in the high half of a byte reads as 16 times the code); int8 codes
// (64 per stage): one int8 MFMA on the 16 codes of the lane's chunk. Sums are exact in int32
// and dequantised (by s_x s_R, and 2^-8 for nibbles) after the K loop, where the
// up-projection follows.
template <class DT, int BM, int BN, bool INTC, bool NIB = true>
__device__ __forceinline__ void gemm_big(const GemmParams& p) {
  typedef MxCfg<BM, BN> C;
  typedef typename DT::T T;
  extern __shared__ __align__(1024) uint8_t smem[];
  // per-wave DMA loads of a stage (INT has no scale words)
  constexpr int LPS = C::A_PER_WAVE + C::B_PER_WAVE + (INTC ? 0 : 1);

  // the wave index is uniform across the wave: kept in a scalar register, so that the LDS
  // destinations of the DMA loads are computed on the scalar unit
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
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

  // ---- per-lane DMA sources (16-byte chunks) for this wave's share of a stage, as 32-bit byte
  // offsets into buffer resources over the four operand arrays (each under 2 GiB, checked by
  // the launcher): the stage advance is the instruction's scalar offset, so a load needs no
  // address arithmetic in the loop, and a resource's range check covers exactly its array.
  int a_off[C::A_PER_WAVE], a_dst[C::A_PER_WAVE];
#pragma unroll
  for (int j = 0; j < C::A_PER_WAVE; j++) {
    const int u = wave + C::NWV * j;  // instruction index: 16 rows x 64 bytes
    const int q = u * 64 + lane;
    const int row = q >> 2, phys = q & 3;
    const int chunk = phys ^ ((row >> 2) & 3);
    int gr = m0 + row;
    gr = gr < p.B ? gr : p.B - 1;
    // MX: 16-row x 128-code tiles, + 1024 per stage; INT: row-major, + 64 per stage
    a_off[j] = INTC ? gr * (int)p.lda + chunk * 16 : ((gr >> 4) * p.kq) * 1024 + (gr & 15) * 64 + chunk * 16;
    a_dst[j] = u * 1024;
  }
  int b_off[C::B_PER_WAVE], b_dst[C::B_PER_WAVE];
#pragma unroll
  for (int j = 0; j < C::B_PER_WAVE; j++) {
    int u = wave + C::NWV * j;
    const bool real = u < C::B_INSTR;
    const int q = (real ? u : 0) * 64 + lane;
    const int row = q >> 2, phys = q & 3;
    const int chunk = phys ^ ((row >> 2) & 3);
    int gr = n0 + row;
    gr = gr < p.npad ? gr : p.npad - 1;
    // MX: tiled, + 1024 per stage; INT: row-major like A, + 64 per stage
    b_off[j] = INTC ? gr * (int)p.ldw + chunk * 16 : (int)mx_code_tile_offset(gr, p.kq) + chunk * 16;
    b_dst[j] = C::A_BYTES + u * 1024;  // u >= B_INSTR lands in the padding after B
  }
  // scales (stage-tiled): waves 0-3 load the 64-row groups 0-3 of the A tile, waves 4-7 those of
  // the B tile, 256 contiguous bytes per stage; groups past the data clamp to the last one
  // (discarded)
  const int sw = wave & 3;
  int ga = (m0 >> 6) + sw;
  ga = ga < p.ascale_groups ? ga : p.ascale_groups - 1;
  const int sa_off = ((ga * p.kq) << 8) + lane * 4;
  int gb = (n0 >> 6) + (64 * sw < BN ? sw : 0);
  gb = gb < (p.npad >> 6) ? gb : (p.npad >> 6) - 1;
  const int sb_off = ((gb * p.kq) << 8) + lane * 4;
  const int s_off_a = C::A_BYTES + C::B_PER_WAVE * C::NWV * 1024;
  const int s_off_b = s_off_a + C::SCALE_BYTES;

  auto issue = [&](int st) {
    uint8_t* base = smem + (st % C::NS) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::A_PER_WAVE; j++)
      buffer_to_lds16(p.acodes, (int)((int64_t)((p.B + 15) & ~15) * p.lda), base + a_dst[j], a_off[j], st * (INTC ? C::SB : 1024));
#pragma unroll
    for (int j = 0; j < C::B_PER_WAVE; j++)
      buffer_to_lds16(p.wcodes, (int)((int64_t)p.npad * (INTC ? p.ldw : (int64_t)p.kq * 64)), base + b_dst[j], b_off[j],
                      st * (INTC ? C::SB : 1024));
    if constexpr (!INTC) {
      if (wave < 4)
        buffer_to_lds4(p.ascales, (int)((int64_t)p.ascale_groups * p.kq * 256), base + s_off_a + sw * 256, sa_off, st * 256);
      else
        buffer_to_lds4(p.wscales, (int)((int64_t)(p.npad >> 6) * p.kq * 256), base + s_off_b + sw * 256, sb_off, st * 256);
    }
  };

  typedef typename std::conditional<INTC, v16i, v16f>::type Acc;
  Acc acc[C::MT][C::NT];
#pragma unroll
  for (int i = 0; i < C::MT; i++)
#pragma unroll
    for (int j = 0; j < C::NT; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0;

  // Operand fragment of one 64-code K slice: A rows and B columns of this wave's tile read
  // from the LDS stage buffer.
  struct Frag {
    v8i a[C::MT], b[C::NT];
  };
  // Scale words of a stage: four E8M0 bytes (one per 32-code block) per row / column.
  struct Scales {
    u32 a[C::MT], b[C::NT];
  };
  // Per-lane byte offsets of the operand reads within a stage buffer, for the two 64-code
  // slices: rows 32 apart share the swizzle (it depends on (row >> 2) & 3), so a wave's MT (NT)
  // rows are one offset plus multiples of 2 KB, immediate offsets of the LDS reads.
  int fa_off[2], fb_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ks++) {
    fa_off[ks] = lds_swz(wm * C::TM + l32, 2 * ks + g);
    fb_off[ks] = C::A_BYTES + lds_swz(wn * C::TN + l32, 2 * ks + g);
  }
  const int sa_lane = s_off_a + (wm * C::TM + l32) * 4, sb_lane = s_off_b + (wn * C::TN + l32) * 4;
  auto read_frag = [&](const uint8_t* base, int ks, Frag& f) {
#pragma unroll
    for (int i = 0; i < C::MT; i++) {
      const v4i a4 = *reinterpret_cast<const v4i*>(base + fa_off[ks] + 2048 * i);
      f.a[i] = v8i{a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < C::NT; j++) {
      const v4i b4 = *reinterpret_cast<const v4i*>(base + fb_off[ks] + 2048 * j);
      f.b[j] = v8i{b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
    }
  };
  // A scale word holds the E8M0 bytes of the stage's four 32-code blocks; lane (l32, g) uses
  // block 2 ks + g in slice ks, so its word is shifted right by 8 g once, and the MFMA picks
  // byte 2 ks of it (the instruction's scale byte select).
  const int gsh = 8 * g;
  auto read_scales = [&](const uint8_t* base, Scales& sc) {
    if constexpr (INTC) return;
#pragma unroll
    for (int i = 0; i < C::MT; i++) sc.a[i] = *reinterpret_cast<const u32*>(base + sa_lane + 128 * i) >> gsh;
#pragma unroll
    for (int j = 0; j < C::NT; j++) sc.b[j] = *reinterpret_cast<const u32*>(base + sb_lane + 128 * j) >> gsh;
  };
  auto mma = [&](const Frag& f, const Scales& sc, auto ks_c) {
    constexpr int KS = decltype(ks_c)::value;
    if constexpr (INTC && !NIB) {
      // lane (l32, g) holds the 16 int8 codes of chunk 2 KS + g: one 32x32x32 MFMA
#pragma unroll
      for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4i{f.a[i][0], f.a[i][1], f.a[i][2], f.a[i][3]},
                                                           v4i{f.b[j][0], f.b[j][1], f.b[j][2], f.b[j][3]}, acc[i][j], 0, 0, 0);
    } else if constexpr (INTC) {
      // lane (l32, g) holds 32 nibble codes of K block 2 KS + g: odd codes (w & 0xF0F0F0F0)
      // and even codes ((w << 4) & 0xF0F0F0F0) as int8 times 16, one 32x32x32 MFMA each
      const v4i m = {(int)0xF0F0F0F0, (int)0xF0F0F0F0, (int)0xF0F0F0F0, (int)0xF0F0F0F0};
      v4i ah[C::MT], al[C::MT], bh[C::NT], bl[C::NT];
#pragma unroll
      for (int i = 0; i < C::MT; i++) {
        const v4i w = {f.a[i][0], f.a[i][1], f.a[i][2], f.a[i][3]};
        ah[i] = w & m;
        al[i] = (w << 4) & m;
      }
#pragma unroll
      for (int j = 0; j < C::NT; j++) {
        const v4i w = {f.b[j][0], f.b[j][1], f.b[j][2], f.b[j][3]};
        bh[j] = w & m;
        bl[j] = (w << 4) & m;
      }
#pragma unroll
      for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ah[i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(al[i], bl[j], acc[i][j], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, 2 * KS, (int)sc.a[i],
                                                                      2 * KS, (int)sc.b[j]);
    }
  };
  typedef std::integral_constant<int, 0> Slice0;
  typedef std::integral_constant<int, 1> Slice1;

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
  constexpr int NM = C::MT * C::NT * (INTC && NIB ? 2 : 1);  // MFMAs per slice
  constexpr int P1 = NM - 1 < NR ? NM - 1 : NR;  // slice-1 reads paired with slice-0 MFMAs
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
  auto up_mma = [&](const UpOps& u, auto& F) {
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
          F[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(u.a[h][i], u.b[h][j], F[i][j], 0, 0, 0);
  };
  // f32 io: down (finished, or the ordered sum of its split-K partials) and L2^T are split
  // into bf16 high and low parts, and down L2 = dh lh + dh ll + dl lh on bf16 MFMAs (the
  // dropped dl ll and the split leave a relative error near 2^-16).
  auto up_f32 = [&](auto& F) {
    for (int kk = 0; kk < p.rp; kk += 16) {
      v8bf ah[C::MT], al[C::MT];
#pragma unroll
      for (int i = 0; i < C::MT; i++) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] = down1_f32(p.down, p.down_part, p.down_chunks, p.B, p.rp, drow[i], kk + 8 * g + e);
        split_bf16x8(v, ah[i], al[i]);
      }
#pragma unroll
      for (int j = 0; j < C::NT; j++) {
        const float* src = reinterpret_cast<const float*>(p.l2t) + (int64_t)bcol[j] * p.rp + kk + 8 * g;
        const float4 l0 = *reinterpret_cast<const float4*>(src), l1 = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        v8bf bh, bl;
        split_bf16x8(v, bh, bl);
#pragma unroll
        for (int i = 0; i < C::MT; i++) {
          F[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh, F[i][j], 0, 0, 0);
          F[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl, F[i][j], 0, 0, 0);
          F[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh, F[i][j], 0, 0, 0);
        }
      }
    }
  };
  // A finished down (no split-K partials) is requested with plain loads before the first stages
  // go out, so their wait before the MFMAs leaves the stages in flight; partials are summed as
  // they arrive, so they are requested after the stages. Every launch has at least two stages.
  UpOps u0;
  const bool up_direct = p.down_chunks <= 1;
  if (!INTC && DT::is_bf16 && p.rp > 0 && up_direct) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int i = 0; i < C::MT; i++)
        u0.a[h][i] = __builtin_bit_cast(
            v8bf, *reinterpret_cast<const v4i*>(reinterpret_cast<const T*>(p.down) + (int64_t)drow[i] * p.rp + 16 * h + 8 * g));
#pragma unroll
      for (int j = 0; j < C::NT; j++)
        u0.b[h][j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(l2t + (int64_t)bcol[j] * p.rp + 16 * h + 8 * g));
    }
  }
  static_assert(C::DIST == 2, "two stages issued here");
  issue(0);
  issue(1);
  if constexpr (!INTC) {
    if constexpr (DT::is_bf16) {
      if (p.rp > 0) {
        if (!up_direct) up_load(u0, 0);
        up_mma(u0, acc);
        for (int kk = 32; kk < p.rp; kk += 32) {
          UpOps u;
          up_load(u, kk);
          up_mma(u, acc);
        }
      }
    } else {
      up_f32(acc);  // requested after the first stages, so its waits cover them too
    }
  }

  wait_stage<LPS, C::DIST + 2>(nst - 1 < C::DIST - 1 ? nst - 1 : C::DIST - 1);
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
    mma(cur0, scur, Slice0());
    // slice 1's reads one per slice-0 MFMA (after the first); reads beyond the MFMAs go last
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int q = 0; q < P1; q++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (NR > P1) __builtin_amdgcn_sched_group_barrier(0x100, NR - P1, 0);
    if constexpr (NM - 1 > P1) __builtin_amdgcn_sched_group_barrier(0x008, NM - 1 - P1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (AHEAD >= 0) {
      wait_vmcnt<LPS * AHEAD>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const uint8_t* nb = smem + ((s + 1) % C::NS) * C::STAGE;
      read_scales(nb, snxt);
      read_frag(nb, 0, nxt0);
    }
    mma(f1, scur, Slice1());
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

  // ---- epilogue on fp32 accumulators F (named acc inside)
  auto finish = [&](auto& acc) {
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
    // 32x32 tile lane (l32, g) holds column l32 of rows 8q + 4g + e (e = 0..3). Each lane rounds
    // rows (r, r+1) of its column into one word (e = 0, 2), neighbouring lanes swap those words
    // (DPP quad_perm [1,0,3,2]), and one byte permute leaves the even lane row r of columns
    // (l32, l32+1) and the odd lane row r+1 of the same two columns: one 4-byte LDS write per
    // pair and no per-pair select.
    if constexpr (!DT::is_bf16) {
      store_f32_tile<BM, BN>(p, acc, smem, t, wm, wn, l32, g, m0, n0);
      return;
    }
    static_assert(BM * BN * 2 <= C::SMEM, "output tile must fit the LDS ring");
    const bool odd = l32 & 1;
    // perm(neighbour, own): bytes 0-3 are the own word, 4-7 the neighbour's; the even lane takes
    // (own.lo, neighbour.lo), the odd lane (neighbour.hi, own.hi)
    const u32 psel = odd ? 0x03020706u : 0x05040100u;
    __syncthreads();
    uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
    uint16_t* wtile = tile + (odd ? BN : 0);
  #pragma unroll
    for (int i = 0; i < C::MT; i++)
  #pragma unroll
      for (int j = 0; j < C::NT; j++) {
        const int c = wn * C::TN + 32 * j + (l32 & ~1);
  #pragma unroll
        for (int q = 0; q < 4; q++)
  #pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const u32 own = pack_bf16x2(acc[i][j][4 * q + e], acc[i][j][4 * q + e + 1]);
            const u32 nb = (u32)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, true);
            const int r = wm * C::TM + 32 * i + 8 * q + 4 * g + e;
            *reinterpret_cast<u32*>(wtile + r * BN + c) = __builtin_amdgcn_perm(nb, own, psel);
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
  };
  if constexpr (INTC) {
    // exact int32 sums (256 times the code products) to fp32, then the up-projection
    v16f facc[C::MT][C::NT];
    const float scl = p.sx[0] * p.sr[0];
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
      for (int j = 0; j < C::NT; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) facc[i][j][v] = ((float)acc[i][j][v] * (NIB ? 0x1p-8f : 1.0f)) * scl;
    if constexpr (DT::is_bf16) {
      for (int kk = 0; kk < p.rp; kk += 32) {
        UpOps u;
        up_load(u, kk);
        up_mma(u, facc);
      }
    } else {
      up_f32(facc);
    }
    finish(facc);
  } else {
    finish(acc);
  }
}

template <class DT, int BM, int BN>
__global__ __launch_bounds__(512) void k_gemm_mx(GemmParams p) {
  gemm_big<DT, BM, BN, false>(p);
}

template <class DT, int BM, int BN, bool NIB>
__global__ __launch_bounds__(512) void k_gemm_int_big(GemmParams p) {
  gemm_big<DT, BM, BN, true, NIB>(p);
}

}  // namespace dev

using namespace dev;

template <class DT, int BM, int BN>
static hipError_t launch_mx_dt(const GemmParams& p, hipStream_t stream) {
  typedef MxCfg<BM, BN> C;
  const int tiles = ((p.B + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mx<DT, BM, BN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    if (e != hipSuccess) return e;
    configured = true;
  }
  return launch_gemm_kernel(k_gemm_mx<DT, BM, BN>, dim3(tiles), dim3(64 * C::NWV), C::SMEM, stream, p);
}

template <class DT, int BM, int BN, bool NIB>
static hipError_t launch_int_big_dt(const GemmParams& p, hipStream_t stream) {
  typedef MxCfg<BM, BN> C;
  const int tiles = ((p.B + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_int_big<DT, BM, BN, NIB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    if (e != hipSuccess) return e;
    configured = true;
  }
  return launch_gemm_kernel(k_gemm_int_big<DT, BM, BN, NIB>, dim3(tiles), dim3(64 * C::NWV), C::SMEM, stream, p);
}

template <int BM, int BN>
static hipError_t launch_int_big_t(const GemmParams& p, bool nib, int dtype, hipStream_t stream) {
  if (nib) return dtype == SVDQ_BF16 ? launch_int_big_dt<BF16, BM, BN, true>(p, stream) : launch_int_big_dt<F32, BM, BN, true>(p, stream);
  return dtype == SVDQ_BF16 ? launch_int_big_dt<BF16, BM, BN, false>(p, stream) : launch_int_big_dt<F32, BM, BN, false>(p, stream);
}

// Compute units of the current device (looked up once per device; 256 if the query fails).
static int64_t device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Index into {128x192, 128x256, 256x192, 256x256} of the tile with the least estimated time:
// rounds of the chip x (10 us + us_per_elem per output element of the tile); 192-wide tiles
// only when N % 192 == 0; the first of equal estimates wins.
static int pick_tile(const GemmParams& p, int64_t cus, double us_per_elem) {
  const int cand[4][2] = {{128, 192}, {128, 256}, {256, 192}, {256, 256}};
  int best = -1;
  double best_t = 0;
  for (int c = 0; c < 4; c++) {
    const int bm = cand[c][0], bn = cand[c][1];
    if (bn == 192 && p.N % 192 != 0) continue;
    const int64_t tiles = ((int64_t)(p.B + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    const int64_t rounds = (tiles + cus - 1) / cus;
    const double t = (double)rounds * (10.0 + us_per_elem * bm * bn);
    if (best < 0 || t < best_t) best = c, best_t = t;
  }
  return best;
}

template <int BM, int BN>
static hipError_t launch_mx_t(const GemmParams& p, int dtype, hipStream_t stream) {
  return dtype == SVDQ_BF16 ? launch_mx_dt<BF16, BM, BN>(p, stream) : launch_mx_dt<F32, BM, BN>(p, stream);
}

// MXFP4 path above decode batches (B > 64), bf16 or f32 io; returns hipErrorNotSupported when
// an operand array is past 2 GiB, so the caller falls back to the general kernel.
bool mx_large_accepts(const GemmParams& p) {
  if (p.B <= 64 || p.kstages < 2 || p.kstages % 2) return false;
  // the operand arrays (activation codes in whole 16-row tiles) are addressed through buffer
  // resources with 32-bit offsets
  const int64_t lim = (int64_t)1 << 31;
  return !((int64_t)((p.B + 15) / 16) * 16 * p.lda >= lim || (int64_t)p.npad * p.kq * 64 >= lim ||
           (int64_t)p.ascale_groups * p.kq * 256 >= lim || (int64_t)(p.npad >> 6) * p.kq * 256 >= lim);
}

hipError_t launch_gemm_mx_large(const GemmParams& p, int dtype, hipStream_t stream) {
  if (!p.acodes_tiled || !mx_large_accepts(p)) return hipErrorNotSupported;
  // Tile shape: the candidate with the least estimated time, rounds of the chip x time per
  // round. A round (every compute unit on one tile) was measured at K = 3072 to take about
  // 10 us + 0.3 ns per output element of the tile: 128x192 17.4 us, 128x256 19.8, 256x192 24.7,
  // 256x256 29.7. So the fewest rounds win first, then the smallest tile (more compute units
  // busy); 192-wide tiles only when N is a multiple of 192. At 4096 rows this picks 256x256 for
  // N = 12288 and 256x192 for N = 3072; at 512 rows or fewer, 128-row tiles.
  const int64_t cus = device_cus();
  switch (pick_tile(p, cus, 0.3e-3)) {
    case 0: return launch_mx_t<128, 192>(p, dtype, stream);
    case 1: return launch_mx_t<128, 256>(p, dtype, stream);
    case 2: return launch_mx_t<256, 192>(p, dtype, stream);
    default: return launch_mx_t<256, 256>(p, dtype, stream);
  }
}

// Per-tensor INT on the large tiles (nibble codes of at most 4 bits, 128 per stage, or int8
// codes of 5-8 bits, 64 per stage); hipErrorNotSupported when the 64 x 64 INT kernel serves
// the shape better, or an operand array is past 2 GiB. Measured at M = N = 4096 (whole calls,
// 4-bit codes): the 64 x 64 kernel takes ~10 us per round of the chip and wins up to two
// rounds (512 rows: 35 us against 39 for the best large tile); from four rounds on the large
// tiles win (1024 rows: 49 us against 55, 4096 rows: 90 against 168). Among the large tiles
// the same estimate as for MXFP4 picks the shape, with twice the MFMA time per output element
// (the int8 rate is half the FP4 rate).
hipError_t launch_gemm_int_big(const GemmParams& p0, int bits, int dtype, hipStream_t stream) {
  if (bits > 8) return hipErrorNotSupported;
  const bool nib = bits <= 4;
  const int64_t cus = device_cus();
  if (((int64_t)(p0.B + 63) / 64) * ((p0.N + 63) / 64) < 4 * cus) return hipErrorNotSupported;
  GemmParams p = p0;
  p.kstages = (int)(p.ldw / 64);  // stages of 64 bytes per row: 128 nibble or 64 int8 codes
  if (p.ldw % 64 || p.kstages < 2 || p.kstages % 2) return hipErrorNotSupported;
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)p.B * p.lda >= lim || (int64_t)p.npad * p.ldw >= lim) return hipErrorNotSupported;
  switch (pick_tile(p, cus, 0.6e-3)) {
    case 0: return launch_int_big_t<128, 192>(p, nib, dtype, stream);
    case 1: return launch_int_big_t<128, 256>(p, nib, dtype, stream);
    case 2: return launch_int_big_t<256, 192>(p, nib, dtype, stream);
    default: return launch_int_big_t<256, 256>(p, nib, dtype, stream);
  }
}

}  // namespace svdq
