// Residual GEMM for per-tensor INT codes on gfx950 (step (c) of the operator):
//   Y = D( s_x s_R (Q(X^) Q(R)) + down L2 )
// with exact integer products on v_mfma_i32_32x32x32_i8 and the up-projection on bf16 (or
// fp32) MFMAs into the dequantised fp32 accumulators.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 3 (per-tensor INT quantisation; Y = (X^ L1) L2 + Q(X^) Q(R)); "flashinfer.gemm.
// svdquant_linear" (the residual GEMM with the up-projection in its epilogue).
//
// Codes of at most 4 bits arrive as two's-complement nibbles (even k in the low nibble; codes of
// 5-8 bits as int8 bytes, which go to the matrix cores unchanged). The matrix cores take
// int8, and a nibble c placed in the high half of a byte reads as the int8 16 c: per 32-bit
// word, w & 0xF0F0F0F0 gives the odd codes and (w << 4) & 0xF0F0F0F0 the even ones, times 16.
// Products are then 256 times the code products (|sum| <= 256 * 64 * K stays far below
// 2^31 for K < 2^17) and the epilogue scales by 2^-8 exactly.
//
// Structure: a 64 x 64 output tile per 256-thread block, so that mid-size batches still give
// hundreds of blocks. K advances in stages of 256 codes (128 bytes per row) that land in a
// ring of LDS buffers through direct global->LDS loads, six stages ahead (all of them when K
// has fewer stages). Within a stage the
// four waves split K: wave w takes the 16-byte chunks 2w and 2w+1 (two 32-code MFMA steps)
// for the whole 64 x 64 tile, which keeps the nibble unpacking below the MFMA time. After
// the K loop the four int32 partial tiles are summed through LDS (exact), and each wave
// finishes one 32 x 32 quadrant (dequantise, up-projection, one rounding); the rounded tile
// is staged in LDS and written with 16-byte stores.
// LDS rows are 128 bytes; chunk c of row r sits at c ^ ((r >> 1) & 7), so the 16-byte reads
// of 16 consecutive rows (one LDS cycle of a ds_read_b128) hit distinct banks.
#include <type_traits>

#include "device_common.h"
#include "gemm_pipe.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

namespace gi {
constexpr int BM = 64, BN = 64;
constexpr int SB = 128;                 // bytes per row per stage (256 codes)
constexpr int A_BYTES = BM * SB, B_BYTES = BN * SB;
constexpr int STAGE = A_BYTES + B_BYTES;  // 16 KB
constexpr int A_PER_WAVE = A_BYTES / 1024 / 4, B_PER_WAVE = B_BYTES / 1024 / 4;  // wave-wide 1 KB loads
constexpr int LOADS_PER_STAGE = A_PER_WAVE + B_PER_WAVE;
constexpr int DIST = 6, NS = DIST + 2;  // stages in flight (96 KB: covers HBM latency), ring depth
constexpr int SMEM = NS * STAGE;          // 128 KB; reused for the partial-tile exchange
static_assert(4 * 4 * 16 * 64 * 4 <= SMEM, "partial tiles must fit the ring");
}  // namespace gi

// Calls f(integral_constant<int, I>) for I = B .. E-1 in order.
template <int B, int E>
struct StaticFor {
  template <class F>
  __device__ static void run(F&& f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>());
      StaticFor<B + 1, E>::run(f);
    }
  }
};

__device__ inline int swz128(int row, int chunk) { return row * gi::SB + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Two words of nibble codes -> one MFMA operand of 16 int8 values (16 x code), in the order
// (even codes of w0, odd of w0, even of w1, odd of w1); A and B use the same order.
__device__ inline v4i nib16(u32 w0, u32 w1) {
  return v4i{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u), (int)((w1 << 4) & 0xF0F0F0F0u),
             (int)(w1 & 0xF0F0F0F0u)};
}

// NIB: codes are nibbles (bits <= 4; 256 codes per 128-byte stage, unpacked to 16 x code);
// otherwise int8 codes (5-8 bits; 128 codes per stage, fed to the matrix cores as stored).
template <class DT, bool NIB>
__global__ __launch_bounds__(256) void k_gemm_int4(GemmParams p) {
  using namespace gi;
  typedef typename DT::T T;
  extern __shared__ __align__(1024) uint8_t smem[];

  // the wave index in a scalar register: the DMA loads' LDS destinations are scalar arithmetic
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // ---- tile order: blocks i, i+8, ... share an XCD; within an XCD the row tiles of one
  // column tile are consecutive, so a weight slice is fetched into that XCD's L2 once
  const int tiles_m = (p.B + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int tid = blockIdx.x;
  if ((ntiles & 7) == 0) tid = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int m0 = (tid % tiles_m) * BM, n0 = (tid / tiles_m) * BN;

  // ---- per-lane DMA sources: wave-wide instruction u covers 8 rows x 128 bytes; 32-bit byte
  // offsets into buffer resources over the two code arrays (each under 2 GiB, checked by the
  // launcher), the stage advance being the instruction's scalar offset
  int a_off[A_PER_WAVE], b_off[B_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; j++) {
    const int q = (wave + 4 * j) * 64 + lane;
    const int row = q >> 3, chunk = (q & 7) ^ ((row >> 1) & 7);
    int gr = m0 + row;
    gr = gr < p.B ? gr : p.B - 1;
    a_off[j] = gr * p.lda + chunk * 16;
  }
#pragma unroll
  for (int j = 0; j < B_PER_WAVE; j++) {
    const int q = (wave + 4 * j) * 64 + lane;
    const int row = q >> 3, chunk = (q & 7) ^ ((row >> 1) & 7);
    int gr = n0 + row;
    gr = gr < p.npad ? gr : p.npad - 1;
    b_off[j] = gr * p.ldw + chunk * 16;
  }
  const int a_bytes = p.B * p.lda, b_bytes = p.npad * p.ldw;
  auto issue = [&](int st) {
    uint8_t* base = smem + (st % NS) * STAGE;
#pragma unroll
    for (int j = 0; j < A_PER_WAVE; j++) buffer_to_lds16(p.acodes, a_bytes, base + (wave + 4 * j) * 1024, a_off[j], st * SB);
#pragma unroll
    for (int j = 0; j < B_PER_WAVE; j++)
      buffer_to_lds16(p.wcodes, b_bytes, base + A_BYTES + (wave + 4 * j) * 1024, b_off[j], st * SB);
  };

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0;

  // Pipeline (DIST stages in flight, NS = DIST + 2 buffers): stage s+DIST is issued at
  // the top of iteration s; the first 16-code half of stage s is unpacked and fed to the
  // matrix cores; then the wave waits for its own loads of stage s+1, one barrier publishes
  // every wave's loads of that stage, and its operands are read from LDS while the second
  // half's MFMAs of stage s run. The barrier of stage s+1 also guarantees that buffer
  // (s-1) % NS, refilled in iteration s+1, is no longer read (its operands were consumed by
  // MFMAs issued before the barrier).
  static_assert(NS >= DIST + 2 && DIST >= 2, "ring layout assumed below");
  const int nst = p.kstages;
  const int ch = 2 * wave + g;  // this lane's 16-byte chunk of every stage
  struct Ops {
    v4i a[2], b[2];
  };
  auto read_stage = [&](int s, Ops& o) {
    const uint8_t* base = smem + (s % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < 2; i++) o.a[i] = *reinterpret_cast<const v4i*>(base + swz128(32 * i + l32, ch));
#pragma unroll
    for (int j = 0; j < 2; j++) o.b[j] = *reinterpret_cast<const v4i*>(base + A_BYTES + swz128(32 * j + l32, ch));
  };
  struct Unp {
    v4i a[2], b[2];
  };
  auto unpack = [&](const Ops& o, int h, Unp& u) {  // the chunk's two 16-code halves are two MFMA K steps
#pragma unroll
    for (int i = 0; i < 2; i++) u.a[i] = nib16((u32)o.a[i][2 * h], (u32)o.a[i][2 * h + 1]);
#pragma unroll
    for (int j = 0; j < 2; j++) u.b[j] = nib16((u32)o.b[j][2 * h], (u32)o.b[j][2 * h + 1]);
  };
  auto mfma4 = [&](const Unp& u) {
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(u.a[i], u.b[j], acc[i][j], 0, 0, 0);
  };
  // one stage; AHEAD = stages issued after s + 1, or -1 for the last stage. The second half's
  // unpacking runs under the first half's MFMAs, the next stage's LDS reads under the second's.
  // int8 codes: one 32-code MFMA step per stage, which runs under the next stage's LDS reads.
  auto stage = [&](int s, const Ops& cur, Ops& nxt, auto ahead_c) {
    constexpr int AHEAD = decltype(ahead_c)::value;
    if constexpr (!NIB) {
      if constexpr (AHEAD >= 0) {
        wait_vmcnt<LOADS_PER_STAGE * AHEAD>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        read_stage(s + 1, nxt);
      }
      Unp u;
#pragma unroll
      for (int i = 0; i < 2; i++) u.a[i] = cur.a[i];
#pragma unroll
      for (int j = 0; j < 2; j++) u.b[j] = cur.b[j];
      mfma4(u);
      if constexpr (AHEAD >= 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the four LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then the MFMAs
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    Unp u0, u1;
    unpack(cur, 0, u0);
    mfma4(u0);
    unpack(cur, 1, u1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (AHEAD >= 0) {
      wait_vmcnt<LOADS_PER_STAGE * AHEAD>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      read_stage(s + 1, nxt);
    }
    mfma4(u1);
    if constexpr (AHEAD >= 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the four LDS reads first
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then the MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  typedef std::integral_constant<int, DIST - 1> Steady;

  Ops oa, ob;
  if (nst >= DIST) {
#pragma unroll
    for (int s = 0; s < DIST; s++) issue(s);
    wait_vmcnt<LOADS_PER_STAGE * (DIST - 1)>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_stage(0, oa);
    // steady state, unrolled by two so that the operands alternate between oa and ob
    int s = 0;
    for (; s + 1 < nst - DIST; s += 2) {
      issue(s + DIST);
      stage(s, oa, ob, Steady());
      issue(s + 1 + DIST);
      stage(s + 1, ob, oa, Steady());
    }
    // the rest: at most one more steady stage, then the last DIST stages (stage nst-DIST+d has
    // DIST-2-d stages issued after the next one; the last has none to read ahead)
    auto drain = [&](Ops& x, Ops& y) {
      StaticFor<0, DIST>::run([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        typedef std::integral_constant<int, DIST - 2 - d> Ahead;
        if constexpr (d & 1)
          stage(nst - DIST + d, y, x, Ahead());
        else
          stage(nst - DIST + d, x, y, Ahead());
      });
    };
    if (s < nst - DIST) {
      issue(s + DIST);
      stage(s, oa, ob, Steady());
      drain(ob, oa);
    } else {
      drain(oa, ob);
    }
  } else {
    // K shorter than DIST stages: all nst stages are issued at once, then consumed in order
    // (stage d has nst-2-d stages issued after the next one)
    auto run_short = [&](auto nc) {
      constexpr int NST = decltype(nc)::value;
      StaticFor<0, NST>::run([&](auto sc) { issue(decltype(sc)::value); });
      wait_vmcnt<LOADS_PER_STAGE * (NST - 1)>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      read_stage(0, oa);
      StaticFor<0, NST>::run([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        typedef std::integral_constant<int, NST - 2 - d> Ahead;
        if constexpr (d & 1)
          stage(d, ob, oa, Ahead());
        else
          stage(d, oa, ob, Ahead());
      });
    };
    static_assert(DIST == 6, "short runs below cover 1 .. DIST - 1 stages");
    switch (nst) {
      case 1: run_short(std::integral_constant<int, 1>()); break;
      case 2: run_short(std::integral_constant<int, 2>()); break;
      case 3: run_short(std::integral_constant<int, 3>()); break;
      case 4: run_short(std::integral_constant<int, 4>()); break;
      default: run_short(std::integral_constant<int, 5>()); break;
    }
  }

  // ---- epilogue operands of this wave's quadrant q = (qi, qj), loaded before the exchange so
  // their latency overlaps it (rank steps of 16 beyond RMAX are loaded when used)
  const int qi = wave >> 1, qj = wave & 1;
  const int row0 = m0 + 32 * qi, col = n0 + 32 * qj + l32;
  int erow = row0 + l32;
  erow = erow < p.B ? erow : p.B - 1;
  const int bcol = col < p.npad ? col : p.npad - 1;
  const T* l2t = reinterpret_cast<const T*>(p.l2t);
  constexpr int RMAX = 4;
  v8bf ub[RMAX];
  Down8Raw<4> ur[RMAX];  // down's entries or split-K partials, summed after the exchange
  float fa[2 * RMAX], fb[2 * RMAX];
  if constexpr (DT::is_bf16) {
#pragma unroll
    for (int r = 0; r < RMAX; r++)
      if (16 * r < p.rp) {
        down8_request<4>(p.down, p.down_part, p.down_chunks, p.B, p.rp, erow, 16 * r + 8 * g, ur[r]);
        ub[r] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(l2t + (int64_t)bcol * p.rp + 16 * r + 8 * g));
      }
  } else {
#pragma unroll
    for (int r = 0; r < 2 * RMAX; r++)
      if (2 * r < p.rp) {
        fa[r] = down1_f32(p.down, p.down_part, p.down_chunks, p.B, p.rp, erow, 2 * r + g);
        fb[r] = l2t[(int64_t)bcol * p.rp + 2 * r + g];
      }
  }

  // ---- exact sum of the four waves' partial tiles; wave q then owns quadrant q. The ring's
  // stages have all been waited for and read, so LDS-only barriers suffice and the epilogue
  // operands requested above stay in flight across the exchange.
  lds_barrier();
  v4i* part = reinterpret_cast<v4i*>(smem);  // [wave][tile][v/4][lane] of 4 int32
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++)
        part[((wave * 4 + 2 * i + j) * 4 + v4) * 64 + lane] =
            v4i{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2], acc[i][j][4 * v4 + 3]};
  lds_barrier();
  v16f f;
  const float scl = p.sx[0] * p.sr[0];
#pragma unroll
  for (int v4 = 0; v4 < 4; v4++) {
    v4i sum = part[((0 * 4 + wave) * 4 + v4) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; w++) sum += part[((w * 4 + wave) * 4 + v4) * 64 + lane];
#pragma unroll
    for (int e = 0; e < 4; e++) f[4 * v4 + e] = ((float)sum[e] * (NIB ? 0x1p-8f : 1.0f)) * scl;
  }

  // ---- up-projection into the fp32 accumulators
  if (p.rp > 0) {
    if constexpr (DT::is_bf16) {
#pragma unroll
      for (int r = 0; r < RMAX; r++)
        if (16 * r < p.rp)
          f = __builtin_amdgcn_mfma_f32_32x32x16_bf16(down8_sum<4>(ur[r], p.down_part, p.down_chunks, p.B, p.rp, erow, 16 * r + 8 * g),
                                                      ub[r], f, 0, 0, 0);
      for (int kk = 16 * RMAX; kk < p.rp; kk += 16) {
        const v8bf av = down8_bf16(p.down, p.down_part, p.down_chunks, p.B, p.rp, erow, kk + 8 * g);
        const v8bf bv = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(l2t + (int64_t)bcol * p.rp + kk + 8 * g));
        f = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, f, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 2 * RMAX; r++)
        if (2 * r < p.rp) f = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[r], fb[r], f, 0, 0, 0);
      for (int kk = 4 * RMAX; kk < p.rp; kk += 2) {
        const float av = down1_f32(p.down, p.down_part, p.down_chunks, p.B, p.rp, erow, kk + g);
        const float bv = l2t[(int64_t)bcol * p.rp + kk + g];
        f = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, f, 0, 0, 0);
      }
    }
  }

  // ---- bias, round once, stage the 64 x 64 tile in LDS and write it with 16-byte stores
  {
    const float bz = bias_at<DT>(p.bias, col, p.N);
#pragma unroll
    for (int v = 0; v < 16; v++) f[v] += bz;
  }
  __syncthreads();  // every wave has read its partial sums
  T* tile = reinterpret_cast<T*>(smem);
#pragma unroll
  for (int v = 0; v < 16; v++)
    tile[(32 * qi + 8 * (v >> 2) + 4 * g + (v & 3)) * BN + 32 * qj + l32] = DT::from_f32(f[v]);
  __syncthreads();
  T* y = reinterpret_cast<T*>(p.y);
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = BN / EPC;        // chunks per tile row
  const bool vec_ok = (p.ldy % EPC == 0) && (((uintptr_t)p.y & 15) == 0);
  for (int c = t; c < BM * CPR; c += 256) {
    const int r = c / CPR, cc = c - r * CPR;
    const int row = m0 + r, c0 = n0 + cc * EPC;
    if (row >= p.B || c0 >= p.N) continue;
    const T* src = tile + r * BN + cc * EPC;
    T* dst = y + (int64_t)row * p.ldy + c0;
    if (vec_ok && c0 + EPC <= p.N) {
      // streaming store (the output is not read again by the operator)
      __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(src), reinterpret_cast<v4i*>(dst));
    } else {
      for (int e = 0; e < EPC && c0 + e < p.N; e++) dst[e] = src[e];
    }
  }
}

}  // namespace dev

using namespace dev;

template <class DT, bool NIB>
static hipError_t launch_int4_t(const GemmParams& p, hipStream_t stream) {
  const int tiles = ((p.B + gi::BM - 1) / gi::BM) * ((p.N + gi::BN - 1) / gi::BN);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_int4<DT, NIB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, gi::SMEM);
    if (e != hipSuccess) return e;
    configured = true;
  }
  return launch_gemm_kernel(k_gemm_int4<DT, NIB>, dim3(tiles), dim3(256), gi::SMEM, stream, p);
}

// Per-tensor INT: nibble codes (at most 4 bits) or int8 codes (5-8 bits), any K; operand
// arrays past 2 GiB fall back to the general kernel.
hipError_t launch_gemm_int4(const GemmParams& p, int bits, int dtype, hipStream_t stream) {
  if (p.kstages < 1) return hipErrorNotSupported;
  // the code arrays are addressed through buffer resources with 32-bit offsets
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)p.B * p.lda >= lim || (int64_t)p.npad * p.ldw >= lim) return hipErrorNotSupported;
  if (bits <= 4) return dtype == SVDQ_BF16 ? launch_int4_t<BF16, true>(p, stream) : launch_int4_t<F32, true>(p, stream);
  return dtype == SVDQ_BF16 ? launch_int4_t<BF16, false>(p, stream) : launch_int4_t<F32, false>(p, stream);
}

}  // namespace svdq
