// Pieces shared by the LDS-ring GEMM kernels: the LDS address space pointer type and direct
// buffer->LDS loads, and waits on the vector-memory counter.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svdq {
namespace dev {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Word 3 of a raw buffer resource on gfx9-family GPUs (no swizzle, 32-bit data format; the
// value AMD's composable_kernel uses for these targets).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Direct loads into LDS through a raw buffer resource over [array, array + bytes): 16 (4) bytes
// per lane from array + voffset + soffset (soffset wave-uniform) to the lane's slot at lds.
__device__ __forceinline__ void buffer_to_lds16(const uint8_t* array, int bytes, uint8_t* lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)array, 0, bytes, kBufferRsrcWord3),
                                           (lds_ptr_t)lds, 16, voffset, soffset, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds4(const uint8_t* array, int bytes, uint8_t* lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)array, 0, bytes, kBufferRsrcWord3),
                                           (lds_ptr_t)lds, 4, voffset, soffset, 0, 0);
}

// s_waitcnt vmcnt(n) for a compile-time n (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until the stage about to be read has landed when up to D later stages may be in flight:
// remaining_after = number of later stages already issued (0 .. D), LPS = loads per stage per
// wave. Loads complete in issue order, so allowing LPS * remaining_after outstanding loads
// leaves the wanted stage done.
template <int LPS, int D>
__device__ inline void wait_stage_upto(int remaining_after) {
  if constexpr (D > 0) {
    if (remaining_after >= D) {
      wait_vmcnt<LPS * D>();
      return;
    }
    wait_stage_upto<LPS, D - 1>(remaining_after);
  } else {
    wait_vmcnt<0>();
  }
}

// The same for a ring of NS buffers read with prefetch distance NS - 2.
template <int LPS, int NS>
__device__ inline void wait_stage(int remaining_after) {
  if constexpr (NS >= 5) {
    if (remaining_after >= 3) {
      wait_vmcnt<LPS * 3>();
      return;
    }
  }
  if constexpr (NS >= 4) {
    if (remaining_after >= 2) {
      wait_vmcnt<LPS * 2>();
      return;
    }
  }
  if (remaining_after >= 1)
    wait_vmcnt<LPS * 1>();
  else
    wait_vmcnt<0>();
}

}  // namespace dev
}  // namespace svdq
