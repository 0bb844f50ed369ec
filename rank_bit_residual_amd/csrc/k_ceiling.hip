// Measured ceilings of the chip, for reporting the operator's kernels against what the hardware
// sustains here as well as against its datasheet peaks (a measurement aid; no page defines it):
//   * k_ceiling_mfma<KIND>: a loop of independent matrix-core instructions on register
//     operands, the kind the residual GEMMs use (KIND 0: v_mfma_scale_f32_32x32x64_f8f6f4 with
//     FP4 operands and unit E8M0 scales; KIND 1: v_mfma_i32_32x32x32_i8). Two waves per SIMD,
//     eight independent accumulators per wave, no memory traffic inside the loop.
//   * k_ceiling_read: a grid-stride stream of 16-byte loads over a buffer (HBM read rate when
//     the buffer is cold).
#include "device_common.h"
#include "launch.h"
#include "../../include/svdq.h"

namespace svdq {
namespace dev {

constexpr int CEIL_ACC = 8;

template <int KIND>
__global__ __launch_bounds__(256) void k_ceiling_mfma(int64_t iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // operands that the compiler cannot fold: lane-dependent bit patterns (FP4 codes or int8
  // values; their magnitude does not change the instruction's timing)
  const int seed = (int)(lane * 0x9E3779B1u) ^ (int)blockIdx.x;
  if constexpr (KIND == 0) {
    const v8i a = {seed, seed ^ 0x11111111, seed ^ 0x22222222, seed ^ 0x33333333, 0, 0, 0, 0};
    const v8i b = {seed ^ 0x44444444, seed ^ 0x55555555, seed ^ 0x66666666, seed ^ 0x77777777, 0, 0, 0, 0};
    v16f acc[CEIL_ACC];
#pragma unroll
    for (int k = 0; k < CEIL_ACC; k++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[k][v] = 0.f;
    for (int64_t it = 0; it < iters; it++) {
#pragma unroll
      for (int k = 0; k < CEIL_ACC; k++)
        acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[k], 4, 4, 0, 127, 0, 127);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < CEIL_ACC; k++) s += acc[k][lane & 15];
    if (lane == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
  } else {
    const v4i a = {seed, seed ^ 0x01010101, seed ^ 0x02020202, seed ^ 0x03030303};
    const v4i b = {seed ^ 0x04040404, seed ^ 0x05050505, seed ^ 0x06060606, seed ^ 0x07070707};
    v16i acc[CEIL_ACC];
#pragma unroll
    for (int k = 0; k < CEIL_ACC; k++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[k][v] = 0;
    for (int64_t it = 0; it < iters; it++) {
#pragma unroll
      for (int k = 0; k < CEIL_ACC; k++) acc[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[k], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int k = 0; k < CEIL_ACC; k++) s += acc[k][lane & 15];
    if (lane == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = (float)s;
  }
}

// XOR of every 16-byte chunk of buf[0, n16) (grid-stride); a lane writes only if its XOR equals
// a value the data never produces, so the loads cannot be dropped and nothing is written.
__global__ __launch_bounds__(256) void k_ceiling_read(const uint4* __restrict__ buf, int64_t n16, uint32_t never,
                                                      uint32_t* __restrict__ out) {
  uint32_t x = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == never) out[blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace dev

namespace {
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}
}  // namespace

hipError_t launch_ceiling(int kind, int64_t arg, const void* buf, size_t bytes, float* out, size_t out_bytes,
                          hipStream_t stream, double* work) {
  using namespace dev;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  if (kind == 0 || kind == 1) {
    // two 256-thread blocks per CU: two waves per SIMD, one float written per wave
    const int blocks = 2 * cus;
    if (arg < 1 || out_bytes < (size_t)blocks * 4 * sizeof(float)) return hipErrorInvalidValue;
    const double per_mfma = kind == 0 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 32;
    *work = (double)blocks * 4 * (double)arg * CEIL_ACC * per_mfma;
    if (kind == 0)
      k_ceiling_mfma<0><<<blocks, 256, 0, stream>>>(arg, out);
    else
      k_ceiling_mfma<1><<<blocks, 256, 0, stream>>>(arg, out);
    return hipGetLastError();
  }
  if (kind == 2) {
    // arg = blocks (of 256 threads); one uint32 per thread may be written (never, in practice)
    if (arg < 1 || arg > (1 << 20) || !buf || bytes < 16 || ((uintptr_t)buf & 15) ||
        out_bytes < (size_t)arg * 256 * sizeof(uint32_t))
      return hipErrorInvalidValue;
    *work = (double)(bytes / 16 * 16);
    k_ceiling_read<<<(unsigned)arg, 256, 0, stream>>>(reinterpret_cast<const uint4*>(buf), (int64_t)(bytes / 16),
                                                     0xDEADBEEFu, reinterpret_cast<uint32_t*>(out));
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace svdq
