// Device-side helpers of libsvdq (gfx950): storage types, the smoothing division, the
// per-tensor INT and per-block MXFP4 quantisers, nibble unpacking and MFMA vector types.
//
// Quantisation follows "SVDQuant Smoothing, Low-rank and Residual Quantization"
// ("Formula and conventions" items 1 and 3: xs = x / scale; s = max|z| / qmax,
// codes = clamp(round half to even(z / s))) and the MXFP4 per-block minmax scheme of the
// msModelSlim SVDQuant guide (step 2). Every value that decides a code is a single IEEE
// binary32 operation (division, bf16 rounding, power-of-two scaling), never a reciprocal
// multiply or a contracted FMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {
namespace dev {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32;
typedef uint64_t u64;
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// ---- storage dtypes ---------------------------------------------------------------------
struct F32 {
  typedef float T;
  static constexpr bool is_bf16 = false;
  __device__ static inline float to_f32(T v) { return v; }
  __device__ static inline T from_f32(float v) { return v; }
};
struct BF16 {
  typedef uint16_t T;  // raw bfloat16 bits
  static constexpr bool is_bf16 = true;
  __device__ static inline float to_f32(T v) { return __uint_as_float((u32)v << 16); }
  // round to nearest, ties to even (inputs are finite)
  __device__ static inline T from_f32(float v) {
    u32 u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (T)(u >> 16);
  }
};

// D(x / s): one IEEE binary32 division, then rounding to the storage dtype.
template <class DT>
__device__ inline float smooth_value(float x, float s) {
  return DT::to_f32(DT::from_f32(x / s));
}

// Correctly rounded x / s from y = RN(1/s) (y = 0 marks a scale outside [2^-90, 2^90]).
// q0 = RN(x y) is refined twice by Newton-Markstein steps q' = RN(q + r y) with the exact
// remainder r = fma(-s, q, x): the first step makes q faithful, the second returns RN(x / s)
// (Markstein 1990, IBM J. Res. Dev. 34(1); Muller et al., Handbook of Floating-Point
// Arithmetic, the FMA-based division theorem). The theorem needs every intermediate in the
// normal range, so tiny, huge or zero quotients (and flagged scales) take the IEEE division.
__device__ inline float div_rn(float x, float s, float y) {
  float q = x * y;
  float r = __builtin_fmaf(-s, q, x);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-s, q, x);
  q = __builtin_fmaf(r, y, q);
  const float aq = fabsf(q), ax = fabsf(x);
  if (!(aq >= 0x1p-90f && aq <= 0x1p90f && ax >= 0x1p-90f)) q = x / s;
  return q;
}

// Round two floats to bfloat16 (nearest, ties to even; v_cvt_pk_bf16_f32), packed low-first.
__device__ inline u32 pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(u32, __builtin_convertvector(f2{a, b}, bf2));
}

// True when t = RN(x * RN(1/s)) may round to a different bfloat16 than RN_f32(x / s):
// t within 3 ulps of a bf16 rounding midpoint (low 16 bits in [0x7FFD, 0x8003]), or t not a
// normal number (zero, subnormal, infinite, NaN) while x is nonzero. The two differ by at
// most 2 ulps when x * RN(1/s) is a normal product of normal factors (each rounding adds at
// most half an ulp of relative error 2^-24, and RN_f32(x / s) half an ulp).
__device__ inline bool bf16_fast_risky(float t, float x) {
  const u32 u = __float_as_uint(t);
  const bool near_mid = (uint16_t)((uint16_t)u + (uint16_t)0x8003u) < (uint16_t)7u;
  // class mask: every class except -normal (bit 3) and +normal (bit 8)
  const bool not_normal = __builtin_amdgcn_classf(t, 0x2F7) && x != 0.f;
  return near_mid || not_normal;
}

// RN_bf16(RN_f32(x / s)) from y = RN(1/s) (0 for a scale outside [2^-90, 2^90]), as a float:
// the product RN(x y) unless bf16_fast_risky flags it, then the correctly rounded division.
__device__ inline float smooth_bf16(float x, float s, float y) {
  float t = x * y;
  if (bf16_fast_risky(t, x)) {
    asm volatile("");  // rarely taken: keep it a branch
    t = div_rn(x, s, y);
  }
  return t;
}

// x / s by q0 = RN(x y) and two Newton-Markstein corrections, without range branches, for
// y = RN(1/s) with s in [2^-90, 2^90]. Rounded on to bfloat16, the result equals
// RN_bf16(RN_f32(x / s)) for every finite bf16 x (including zeros and subnormals), except that
// a quotient that overflows comes out as NaN instead of +-infinity; callers replace those.
// The sign of x is restored for zeros (the corrections would turn -0 into +0).
__device__ inline float div_markstein(float x, float s, float y) {
  float q = x * y;
  float r = __builtin_fmaf(-s, q, x);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-s, q, x);
  q = __builtin_fmaf(r, y, q);
  return __uint_as_float(__float_as_uint(q) | (__float_as_uint(x) & 0x80000000u));
}

// ---- MXFP4 ------------------------------------------------------------------------------
// Shared exponent of a 32-element block from its max magnitude a: the smallest e with
// a <= 6 * 2^e, clamped to [-127, 127] (E8M0 byte = e + 127). For normal a = 1.m * 2^E the
// answer is E - 2, or E - 1 when 1.m > 1.5; a below 2^-126 (including 0) gives -127.
__device__ inline int mx_exponent(float a) {
  const u32 u = __float_as_uint(a);
  const int be = (int)(u >> 23);
  if (be == 0) return -127;
  const int e = be - 129 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^e as a float for e in [-127, 127] (2^-127 is subnormal).
__device__ inline float pow2f(int e) {
  return e >= -126 ? __uint_as_float((u32)(e + 127) << 23) : __uint_as_float(0x00400000u);
}
// Eight E2M1 codes of v[0..7] / 2^e packed into one word (element 2p in the low nibble of
// byte p). v_cvt_scalef32_pk_fp4_f32 divides by the power-of-two scale and rounds to the
// nearest E2M1 value, ties to the even code, keeping the sign of zero.
__device__ inline u32 fp4_pack8(const float* v, float scale) {
  u32 r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], scale, 3);
  return r;
}

// The same from eight bfloat16 values (four packed pairs, element 2p low in pair p):
// v_cvt_scalef32_pk_fp4_bf16 converts the exact bf16 values with the same rounding.
__device__ inline u32 fp4_pack8_bf16(const u32* pairs, float scale) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  u32 r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf2, pairs[0]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf2, pairs[1]), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf2, pairs[2]), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf2, pairs[3]), scale, 3);
  return r;
}

// Stage-tiled E8M0 layout used inside the library: for each group of 64 rows and each
// 128-code K stage, the 64 rows' four block bytes are contiguous (256 bytes), so one wave
// loads a stage's scales for 64 rows with four 64-byte requests.
__host__ __device__ inline int64_t mx_scale_tiled_index(int64_t row, int64_t kb, int64_t kq) {
  return (((row >> 6) * kq + (kb >> 2)) << 8) + ((row & 63) << 2) + (kb & 3);
}
// Prepared MXFP4 residual codes come in 1 KB tiles (16 columns x 64 bytes = 128 codes):
// byte j of column n at ((n/16) * kq + j/64) * 1024 + (n%16) * 64 + j%64. Offset of
// column n's first K step; step s adds 1024 * s.
__host__ __device__ inline int64_t mx_code_tile_offset(int64_t n, int64_t kq) {
  return (((n >> 4) * kq) << 10) + ((n & 15) << 6);
}

// ---- per-tensor INT ---------------------------------------------------------------------
// clamp(round_half_even(z / s), -qmax, qmax) with an IEEE division; s == 0 gives code 0.
__device__ inline int int_code(float z, float s, float qmax) {
  if (s == 0.f) return 0;
  const float r = __builtin_rintf(z / s);
  return (int)fminf(fmaxf(r, -qmax), qmax);
}

// Sign-extend eight 4-bit two's-complement codes (one word, code j in nibble j) into two
// words of int8 lanes: lo = codes 0,2,4,6 and hi = codes 1,3,5,7. The order inside a lane
// is irrelevant to the matrix cores as long as both operands use it.
__device__ inline void unpack_nibbles(u32 w, u32& lo, u32& hi) {
  const u32 e = w & 0x0F0F0F0Fu, o = (w >> 4) & 0x0F0F0F0Fu;
  // per byte t in [0,15]: ((t ^ 8) | 0x80) - 8 never borrows; ^ 0x80 yields int8(t - 16*(t>=8))
  lo = (((e ^ 0x08080808u) | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
  hi = (((o ^ 0x08080808u) | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
}

// ---- the down-projection operand of the GEMM epilogues -----------------------------------
// Split-K partials of down are stored per chunk in groups of 16 rank columns: chunk c holds
// [rp / 16][B][16] f32, so the entries (row, k) of one 16-column group for consecutive rows are
// contiguous (a wave reading 16 rows x 16 columns reads one kilobyte). Chunks are B * rp apart.
__device__ inline int64_t part_index(int B, int row, int k) { return ((int64_t)(k >> 4) * B + row) * 16 + (k & 15); }

// Eight consecutive entries down[row][k .. k+8) as bf16 (the operand of the up-projection
// MFMAs): read directly, or, when the activation kernel split K over `chunks` blocks, the sum
// of the f32 partials in chunk order 0, 1, ..., rounded once to bf16 (the same value the
// unsplit kernel would store).
// The operands of down8_bf16_pf, requested by down8_request and summed by down8_sum, so that a
// caller can put other work (or other requests) between the two.
template <int PF>
struct Down8Raw {
  float4 lo[PF], hi[PF];
};

template <int PF>
__device__ inline void down8_request(const void* down, const float* part, int chunks, int B, int rp, int row, int k,
                                     Down8Raw<PF>& r) {
  if (chunks <= 1) {  // the eight bf16 entries, as bits
    r.lo[0] = *reinterpret_cast<const float4*>(reinterpret_cast<const uint16_t*>(down) + (int64_t)row * rp + k);
    return;
  }
  const float* src = part + part_index(B, row, k);  // k % 16 is 0 or 8: the eight entries are contiguous
  const int64_t stride = (int64_t)B * rp;
  // the first PF chunks are requested together (indices past the last chunk reload the last one)
#pragma unroll
  for (int c = 0; c < PF; c++) {
    const int cc = c < chunks ? c : chunks - 1;
    r.lo[c] = *reinterpret_cast<const float4*>(src + cc * stride);
    r.hi[c] = *reinterpret_cast<const float4*>(src + cc * stride + 4);
  }
}

// The sum runs in chunk order; chunks past PF are loaded one after another. A requested chunk
// past the last adds -0.0, which leaves every sum unchanged, so the adds need no branch (a
// branch per chunk let the compiler sink that chunk's loads behind the waits for the others).
template <int PF>
__device__ inline v8bf down8_sum(const Down8Raw<PF>& r, const float* part, int chunks, int B, int rp, int row, int k) {
  if (chunks <= 1) return __builtin_bit_cast(v8bf, r.lo[0]);
  float s[8] = {r.lo[0].x, r.lo[0].y, r.lo[0].z, r.lo[0].w, r.hi[0].x, r.hi[0].y, r.hi[0].z, r.hi[0].w};
#pragma unroll
  for (int c = 1; c < PF; c++) {
    const bool on = c < chunks;
    s[0] += on ? r.lo[c].x : -0.0f; s[1] += on ? r.lo[c].y : -0.0f; s[2] += on ? r.lo[c].z : -0.0f; s[3] += on ? r.lo[c].w : -0.0f;
    s[4] += on ? r.hi[c].x : -0.0f; s[5] += on ? r.hi[c].y : -0.0f; s[6] += on ? r.hi[c].z : -0.0f; s[7] += on ? r.hi[c].w : -0.0f;
  }
  const float* src = part + part_index(B, row, k);
  const int64_t stride = (int64_t)B * rp;
  for (int c = PF; c < chunks; c++) {
    const float4 a = *reinterpret_cast<const float4*>(src + c * stride), b = *reinterpret_cast<const float4*>(src + c * stride + 4);
    s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w; s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
  }
  return __builtin_bit_cast(v8bf, v4i{(int)pack_bf16x2(s[0], s[1]), (int)pack_bf16x2(s[2], s[3]),
                                      (int)pack_bf16x2(s[4], s[5]), (int)pack_bf16x2(s[6], s[7])});
}

template <int PF>
__device__ inline v8bf down8_bf16_pf(const void* down, const float* part, int chunks, int B, int rp, int row, int k) {
  Down8Raw<PF> r;
  down8_request<PF>(down, part, chunks, B, rp, row, k, r);
  return down8_sum<PF>(r, part, chunks, B, rp, row, k);
}

__device__ inline v8bf down8_bf16(const void* down, const float* part, int chunks, int B, int rp, int row, int k) {
  return down8_bf16_pf<1>(down, part, chunks, B, rp, row, k);
}

// One entry down[row][k] as f32 (f32 io): direct, or the ordered sum of the partials.
__device__ inline float down1_f32(const void* down, const float* part, int chunks, int B, int rp, int row, int k) {
  if (chunks <= 1) return reinterpret_cast<const float*>(down)[(int64_t)row * rp + k];
  const float* src = part + part_index(B, row, k);
  float s = src[0];
  for (int c = 1; c < chunks; c++) s += src[(int64_t)c * B * rp];
  return s;
}

// ---- output bias ----------------------------------------------------------------------
// bias[min(col, N - 1)] as f32, or 0 without a bias (columns past N are never stored).
template <class DT>
__device__ inline float bias_at(const void* bias, int col, int N) {
  if (!bias) return 0.f;
  return DT::to_f32(reinterpret_cast<const typename DT::T*>(bias)[col < N ? col : N - 1]);
}

// A workgroup barrier for LDS hand-offs only: the wave's own LDS operations complete
// (lgkmcnt(0)), then s_barrier. Unlike __syncthreads it does not wait for outstanding global
// loads and stores (vmcnt counts both), so those stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- wave / block reductions ------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace dev
}  // namespace svdq
