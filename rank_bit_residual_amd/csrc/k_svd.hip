// Device backend for the one-time truncated SVD: the large products of the randomized
// subspace iteration (Halko, Martinsson & Tropp 2011, Algorithm 4.4) with the smoothed weight,
// in float64 on the GPU. The small dense steps (Gram-Schmidt of the panels, the Jacobi
// Rayleigh-Ritz step) stay on the host.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 2 (left @ right is a best rank-r approximation from a truncated SVD; any equivalent
// factorisation is accepted).
//
// k_panel_product<KIND>: C[c][o] = sum_t P[c][t] * A(t, o) for a panel P of k columns; KIND 0
// reads A(t, o) = A[t][o] (t < M, o < N), KIND 1 reads A(t, o) = A[o][t] (t < N, o < M). A
// 256-thread block owns 16 panel columns x 64 outputs and walks t in chunks of 64, staging the
// A chunk (converted to float64) and the P chunk in LDS; each thread accumulates 4 outputs in
// float64 in a fixed order, so results do not depend on the launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "host_svd.h"
#include "svdq_internal.h"

namespace svdq {
namespace dev {

constexpr int PC = 16, PO = 64, PT = 64;  // panel columns, outputs, reduction chunk per block

template <int KIND>
__global__ __launch_bounds__(256) void k_panel_product(const float* __restrict__ A, int64_t lda, int T, int O, int k,
                                                       const double* __restrict__ P, double* __restrict__ C) {
  __shared__ double sa[PT][PO + 1];
  __shared__ double sp[PC][PT + 1];
  const int t = threadIdx.x;
  const int o0 = blockIdx.x * PO, c0 = blockIdx.y * PC;
  const int oc = t & 63, cq = t >> 6;  // this thread: output o0 + oc, panel columns c0 + cq + 4 j
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int t0 = 0; t0 < T; t0 += PT) {
    // A chunk [PT x PO]: KIND 0 rows t (contiguous along o), KIND 1 rows o (contiguous along t)
    for (int q = t; q < PT * PO; q += 256) {
      int tt, oo;
      if (KIND == 0) {
        tt = q / PO;
        oo = q % PO;
      } else {
        oo = q / PT;
        tt = q % PT;
      }
      const int ta = t0 + tt, oa = o0 + oo;
      float v = 0.f;
      if (ta < T && oa < O) v = KIND == 0 ? A[(int64_t)ta * lda + oa] : A[(int64_t)oa * lda + ta];
      sa[tt][oo] = (double)v;
    }
    for (int q = t; q < PC * PT; q += 256) {
      const int cc = q / PT, tt = q % PT;
      const int ca = c0 + cc, ta = t0 + tt;
      sp[cc][tt] = (ca < k && ta < T) ? P[(int64_t)ca * T + ta] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int tt = 0; tt < PT; tt++) {
      const double a = sa[tt][oc];
#pragma unroll
      for (int j = 0; j < 4; j++) acc[j] = __builtin_fma(sp[cq + 4 * j][tt], a, acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int c = c0 + cq + 4 * j, o = o0 + oc;
    if (c < k && o < O) C[(int64_t)c * O + o] = acc[j];
  }
}

// The panel products with A kept on the device: A [M x N] float32 is uploaded once; each
// product uploads P, runs one kernel and downloads C on `stream`, synchronously.
class DevicePanels final : public host::PanelProducts {
 public:
  DevicePanels(const float* A_host, int64_t M, int64_t N, int64_t k, uint8_t* ws, hipStream_t s)
      : M_(M), N_(N), k_(k), s_(s) {
    const int64_t L = M > N ? M : N;
    A_ = reinterpret_cast<float*>(ws);
    P_ = reinterpret_cast<double*>(ws + round_up(M * N * 4, kAlign));
    C_ = reinterpret_cast<double*>(ws + round_up(M * N * 4, kAlign) + round_up(k * L * 8, kAlign));
    note(hipMemcpyAsync(A_, A_host, (size_t)(M * N * 4), hipMemcpyHostToDevice, s_));
  }
  void product(int kind, int64_t k, const double* P, double* C) override {
    const int64_t T = kind == 0 ? M_ : N_, O = kind == 0 ? N_ : M_;
    if (err_ == hipSuccess) {
      note(hipMemcpyAsync(P_, P, (size_t)(k * T * 8), hipMemcpyHostToDevice, s_));
      const dim3 grid((unsigned)((O + PO - 1) / PO), (unsigned)((k + PC - 1) / PC));
      if (kind == 0)
        k_panel_product<0><<<grid, 256, 0, s_>>>(A_, N_, (int)T, (int)O, (int)k, P_, C_);
      else
        k_panel_product<1><<<grid, 256, 0, s_>>>(A_, N_, (int)T, (int)O, (int)k, P_, C_);
      note(hipGetLastError());
      note(hipMemcpyAsync(C, C_, (size_t)(k * O * 8), hipMemcpyDeviceToHost, s_));
      note(hipStreamSynchronize(s_));
    }
    if (err_ != hipSuccess)
      for (int64_t i = 0; i < k * O; i++) C[i] = 0.0;  // the caller reports err_
  }
  hipError_t error() const { return err_; }
  static size_t bytes(int64_t M, int64_t N, int64_t k) {
    const int64_t L = M > N ? M : N;
    return (size_t)(round_up(M * N * 4, kAlign) + 2 * round_up(k * L * 8, kAlign));
  }

 private:
  void note(hipError_t e) {
    if (err_ == hipSuccess && e != hipSuccess) err_ = e;
  }
  int64_t M_, N_, k_;
  hipStream_t s_;
  float* A_ = nullptr;
  double *P_ = nullptr, *C_ = nullptr;
  hipError_t err_ = hipSuccess;
};

}  // namespace dev

size_t device_panels_bytes(int64_t M, int64_t N, int64_t k) { return dev::DevicePanels::bytes(M, N, k); }

int run_split_on_device(const float* A, int64_t M, int64_t N, int64_t r, void* workspace, void* stream, double* L1,
                        double* L2) {
  const int64_t k = host::randomized_panel_columns(M, N, r);
  if (k == 0) {
    host::truncated_svd(A, M, N, N, r, L1, L2);
    return 0;
  }
  dev::DevicePanels panels(A, M, N, k, reinterpret_cast<uint8_t*>(workspace), (hipStream_t)stream);
  host::truncated_svd(A, M, N, N, r, L1, L2, &panels);
  return (int)panels.error();
}

}  // namespace svdq
