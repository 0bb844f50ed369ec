// Truncated SVD of the smoothed weight on the GPU, for the one-time preparation: the randomized
// subspace iteration (Halko, Martinsson & Tropp 2011, Algorithm 4.4: k = rank + 32 columns, 16
// power iterations) and its Rayleigh-Ritz step run on the device in float64; the host only
// factors k x k Gram matrices (Cholesky) and orders k singular values.
//
// Pages: "SVDQuant Smoothing, Low-rank and Residual Quantization", "Formula and conventions"
// item 2 (left @ right is a best rank-r approximation from a truncated SVD; any equivalent
// factorisation is accepted).
//
// Device steps, all float64:
//  * panel products with the weight A [M x N] (float32, kept on the device): Z = A^T Q and
//    Q = A Z on v_mfma_f64_16x16x4_f64 (k_panel_mfma);
//  * orthonormalisation of a panel P [T x k] by Cholesky-QR, twice: G = P^T P on the same MFMA
//    kernel, G + s I = R^T R on the host (s = 1e-13 trace(G) / k keeps a rank-deficient panel
//    factorisable), P <- P R^-1 on the device (k_panel_times);
//  * Rayleigh-Ritz: B = Q^T A [k x N], one-sided Jacobi on B's rows with the round-robin pair
//    order, one kernel per round (k_jacobi_round), the rotations accumulated in J [k x k];
//  * the factors: L1 = Q (J_r diag(sigma_r)), L2 = rows of the rotated B over sigma_r.
// Every reduction runs in a fixed order, so the result does not depend on timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "host_svd.h"
#include "svdq_internal.h"

namespace svdq {
namespace dev {

typedef double v4d __attribute__((ext_vector_type(4)));

// C[c][o] = sum_t P[c * T + t] * Y(t, o) for c < k, o < O (C row-major [k x O], i.e. the
// column-major panel [O x k] of the product's columns). YK 0: Y(t, o) = A[t * lda + o];
// YK 1: Y(t, o) = A[o * lda + t] (A float32); YK 2: Y(t, o) = Yd[o * T + t] (a float64 panel).
// A 256-thread block owns 32 panel columns x 64 outputs and walks t in chunks of 32 staged in
// LDS; each wave runs two 16 x 16 output tiles on v_mfma_f64_16x16x4_f64, whose operands are:
// A[i][q] from lane i + 16 q, B[q][j] from lane j + 16 q, and D[i][j] in lane j + 16 (i % 4),
// slot i / 4.
constexpr int PBC = 32, PBO = 64, PTC = 32;

template <int YK>
__global__ __launch_bounds__(256) void k_panel_mfma(const float* __restrict__ A, int64_t lda, const double* __restrict__ Yd,
                                                    int T, int O, int k, const double* __restrict__ P,
                                                    double* __restrict__ C) {
  __shared__ double sp[PBC][PTC + 1];
  __shared__ double sy[PTC][PBO + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int o0 = blockIdx.x * PBO, c0 = blockIdx.y * PBC;
  v4d acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  for (int t0 = 0; t0 < T; t0 += PTC) {
    for (int q = tid; q < PBC * PTC; q += 256) {
      const int cc = q / PTC, tt = q % PTC;
      const int ca = c0 + cc, ta = t0 + tt;
      sp[cc][tt] = (ca < k && ta < T) ? P[(int64_t)ca * T + ta] : 0.0;
    }
    for (int q = tid; q < PTC * PBO; q += 256) {
      int tt, oo;
      if (YK == 0) {
        tt = q / PBO;
        oo = q % PBO;
      } else {
        oo = q / PTC;
        tt = q % PTC;
      }
      const int ta = t0 + tt, oa = o0 + oo;
      double v = 0.0;
      if (ta < T && oa < O) {
        if (YK == 0) v = (double)A[(int64_t)ta * lda + oa];
        if (YK == 1) v = (double)A[(int64_t)oa * lda + ta];
        if (YK == 2) v = Yd[(int64_t)oa * T + ta];
      }
      sy[tt][oo] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < PTC; kk += 4) {
      const int q = kk + (lane >> 4);
      const double b = sy[q][16 * w + (lane & 15)];
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(sp[lane & 15][q], b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(sp[16 + (lane & 15)][q], b, acc1, 0, 0, 0);
    }
    __syncthreads();
  }
  const int o = o0 + 16 * w + (lane & 15);
  if (o < O) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int c = c0 + (lane >> 4) + 4 * v;
      if (c < k) C[(int64_t)c * O + o] = acc0[v];
      if (c + 16 < k) C[(int64_t)(c + 16) * O + o] = acc1[v];
    }
  }
}

// out[c * T + t] = sum_{a < k (a <= c when UPPER)} P[a * T + t] * S[a * ld + c], for c < nc: the
// panel P [T x k] times a small k x nc matrix S (row-major, row stride ld). A 64-thread block
// stages the k values of its 64 rows in LDS; S is read wave-uniformly.
template <bool UPPER>
__global__ __launch_bounds__(64) void k_panel_times(const double* __restrict__ P, int T, int k, const double* __restrict__ S,
                                                    int ld, int nc, double* __restrict__ out) {
  extern __shared__ double sp[];  // [k][64]
  const int lane = threadIdx.x;
  const int t = blockIdx.x * 64 + lane;
  for (int a = 0; a < k; a++) sp[a * 64 + lane] = t < T ? P[(int64_t)a * T + t] : 0.0;
  __syncthreads();
  if (t >= T) return;
  for (int c = 0; c < nc; c++) {
    const int amax = UPPER ? (c + 1 < k ? c + 1 : k) : k;
    double s = 0.0;
    for (int a = 0; a < amax; a++) s = __builtin_fma(sp[a * 64 + lane], S[(int64_t)a * ld + c], s);
    out[(int64_t)c * T + t] = s;
  }
}

// Fixed-order sum over a 256-thread block; every thread receives the result.
__device__ inline double block_sum256(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// One round of the one-sided Jacobi method on the k rows of B [k x n] (row stride n): block b
// takes the pair (pairs[2b], pairs[2b+1]) (an index >= k is a bye), and rotates the two rows,
// and the same two columns of J (column c at J + c * k), when they are not orthogonal to
// relative tolerance tol (the same rotation as the host's jacobi_columns). Counts rotations.
__global__ __launch_bounds__(256) void k_jacobi_round(double* __restrict__ Bm, int64_t n, int k, double* __restrict__ J,
                                                      const int* __restrict__ pairs, double tol, int* __restrict__ rotated) {
  __shared__ double sh[256];
  int p = pairs[2 * blockIdx.x], q = pairs[2 * blockIdx.x + 1];
  if (p >= k || q >= k) return;
  if (p > q) {
    const int s = p;
    p = q;
    q = s;
  }
  double* x = Bm + (int64_t)p * n;
  double* y = Bm + (int64_t)q * n;
  double a = 0.0, b = 0.0, g = 0.0;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const double xv = x[j], yv = y[j];
    a = __builtin_fma(xv, xv, a);
    b = __builtin_fma(yv, yv, b);
    g = __builtin_fma(xv, yv, g);
  }
  const double alpha = block_sum256(a, sh), beta = block_sum256(b, sh), gamma = block_sum256(g, sh);
  if (!(fabs(gamma) > tol * sqrt(alpha * beta))) return;
  const double zeta = (beta - alpha) / (2.0 * gamma);
  const double t = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + hypot(1.0, zeta));
  const double c = 1.0 / sqrt(1.0 + t * t), s = c * t;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const double xv = x[j], yv = y[j];
    x[j] = c * xv - s * yv;
    y[j] = s * xv + c * yv;
  }
  double* jp = J + (int64_t)p * k;
  double* jq = J + (int64_t)q * k;
  for (int i = threadIdx.x; i < k; i += 256) {
    const double xv = jp[i], yv = jq[i];
    jp[i] = c * xv - s * yv;
    jq[i] = s * xv + c * yv;
  }
  if (threadIdx.x == 0) atomicAdd(rotated, 1);
}

// norms[c] = || row c of B [k x n] ||_2 (fixed-order sums)
__global__ __launch_bounds__(256) void k_row_norms(const double* __restrict__ Bm, int64_t n, double* __restrict__ norms) {
  __shared__ double sh[256];
  const double* x = Bm + (int64_t)blockIdx.x * n;
  double a = 0.0;
  for (int64_t j = threadIdx.x; j < n; j += 256) a = __builtin_fma(x[j], x[j], a);
  a = block_sum256(a, sh);
  if (threadIdx.x == 0) norms[blockIdx.x] = sqrt(a);
}

// J = identity [k x k]
__global__ void k_identity(double* J, int k) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)k * k) J[i] = (i / k == i % k) ? 1.0 : 0.0;
}

// Deterministic standard normals for the starting panel (splitmix64 + Box-Muller, as the host
// route draws them).
struct Normal {
  uint64_t state;
  bool have = false;
  double spare = 0;
  explicit Normal(uint64_t seed) : state(seed) {}
  uint64_t next() {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
  double operator()() {
    if (have) {
      have = false;
      return spare;
    }
    const double u = uniform(), v = uniform();
    const double r = std::sqrt(-2.0 * std::log(u)), t = 6.283185307179586 * v;
    spare = r * std::sin(t);
    have = true;
    return r * std::cos(t);
  }
};

// Workspace of the device route: A (float32), three panels of max(M, N) x k, B [k x N], and the
// small k x k matrices, the pair schedule and the rotation counter.
struct SvdWorkspace {
  float* A;
  double *p0, *p1, *p2, *Bm, *G, *S, *J, *norms;
  int *pairs, *counter;
  static int64_t layout(int64_t M, int64_t N, int64_t k, int64_t r, uint8_t* base, SvdWorkspace* w) {
    const int64_t L = std::max(M, N), np = k + (k & 1);
    int64_t o = 0;
    auto take = [&](int64_t bytes) {
      const int64_t at = o;
      o = round_up(o + bytes, kAlign);
      return base ? base + at : nullptr;
    };
    uint8_t* a = take(M * N * 4);
    uint8_t* p0 = take(L * k * 8);
    uint8_t* p1 = take(L * k * 8);
    uint8_t* p2 = take(L * k * 8);
    uint8_t* bm = take(k * N * 8);
    uint8_t* g = take(k * k * 8);
    uint8_t* s = take(k * std::max(k, r) * 8);
    uint8_t* j = take(k * k * 8);
    uint8_t* nr = take(k * 8);
    uint8_t* pr = take((np - 1) * np * 4);
    uint8_t* ct = take(4);
    if (w) {
      w->A = reinterpret_cast<float*>(a);
      w->p0 = reinterpret_cast<double*>(p0);
      w->p1 = reinterpret_cast<double*>(p1);
      w->p2 = reinterpret_cast<double*>(p2);
      w->Bm = reinterpret_cast<double*>(bm);
      w->G = reinterpret_cast<double*>(g);
      w->S = reinterpret_cast<double*>(s);
      w->J = reinterpret_cast<double*>(j);
      w->norms = reinterpret_cast<double*>(nr);
      w->pairs = reinterpret_cast<int*>(pr);
      w->counter = reinterpret_cast<int*>(ct);
    }
    return o;
  }
};

class DeviceSvd {
 public:
  DeviceSvd(const float* A_host, int64_t M, int64_t N, int64_t k, int64_t r, uint8_t* ws, hipStream_t s)
      : M_(M), N_(N), k_(k), r_(r), s_(s) {
    SvdWorkspace::layout(M, N, k, r, ws, &w_);
    // k_panel_times stages k x 64 float64 values (up to kMaxDeviceK: 128 KB)
    note(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_panel_times<true>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxDeviceK * 64 * 8)));
    note(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_panel_times<false>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxDeviceK * 64 * 8)));
    note(hipMemcpyAsync(w_.A, A_host, (size_t)(M * N * 4), hipMemcpyHostToDevice, s_));
  }
  hipError_t error() const { return err_; }

  // The randomized route; L1 [M x r] and L2 [r x N] row-major on the host.
  void run(int power_iters, double* L1, double* L2) {
    const int64_t k = k_;
    // starting panel: Omega [N x k] of standard normals, drawn as the host route draws it
    std::vector<double> om((size_t)(N_ * k));
    Normal rng(0x5EEDull + (uint64_t)M_ * 1000003ull + (uint64_t)N_);
    for (auto& v : om) v = rng();
    note(hipMemcpyAsync(w_.p1, om.data(), om.size() * 8, hipMemcpyHostToDevice, s_));
    double* q = w_.p0;  // Q [M x k]
    double* z = w_.p1;  // Z [N x k]
    product(1, z, q);   // Q = A Omega
    orthonormalize(q, M_);
    for (int it = 0; it < power_iters; it++) {
      product(0, q, z);  // Z = A^T Q
      orthonormalize(z, N_);
      product(1, z, q);  // Q = A Z
      orthonormalize(q, M_);
    }
    product(0, q, w_.Bm);  // B = Q^T A, [k x N]
    jacobi();
    // singular values: norms of B's rotated rows, in decreasing order (ties by index)
    std::vector<double> sigma((size_t)k), J((size_t)(k * k));
    launch_ok();
    if (!err_) k_row_norms<<<(unsigned)k, 256, 0, s_>>>(w_.Bm, N_, w_.norms);
    launch_ok();
    note(hipMemcpyAsync(sigma.data(), w_.norms, (size_t)k * 8, hipMemcpyDeviceToHost, s_));
    note(hipMemcpyAsync(J.data(), w_.J, (size_t)(k * k) * 8, hipMemcpyDeviceToHost, s_));
    note(hipStreamSynchronize(s_));
    if (err_) return;
    std::vector<int64_t> ord((size_t)k);
    std::iota(ord.begin(), ord.end(), 0);
    std::stable_sort(ord.begin(), ord.end(), [&](int64_t a, int64_t b) { return sigma[a] > sigma[b]; });
    // L1 = Q (J_r diag(sigma_r)) on the device; L2 = B's rows / sigma on the host
    const int64_t r = r_;
    std::vector<double> S((size_t)(k * r));
    for (int64_t t = 0; t < r; t++)
      for (int64_t a = 0; a < k; a++) S[a * r + t] = J[ord[t] * k + a] * sigma[ord[t]];
    note(hipMemcpyAsync(w_.S, S.data(), S.size() * 8, hipMemcpyHostToDevice, s_));
    double* l1d = w_.p2;
    if (!err_)
      k_panel_times<false><<<(unsigned)((M_ + 63) / 64), 64, (size_t)k * 64 * 8, s_>>>(q, (int)M_, (int)k, w_.S, (int)r,
                                                                                     (int)r, l1d);
    launch_ok();
    std::vector<double> l1((size_t)(M_ * r)), bm((size_t)(k * N_));
    note(hipMemcpyAsync(l1.data(), l1d, l1.size() * 8, hipMemcpyDeviceToHost, s_));
    note(hipMemcpyAsync(bm.data(), w_.Bm, bm.size() * 8, hipMemcpyDeviceToHost, s_));
    note(hipStreamSynchronize(s_));
    if (err_) return;
    for (int64_t i = 0; i < M_; i++)
      for (int64_t t = 0; t < r; t++) L1[i * r + t] = l1[t * M_ + i];
    for (int64_t t = 0; t < r; t++) {
      const double sg = sigma[ord[t]];
      const double* row = bm.data() + ord[t] * N_;
      for (int64_t j = 0; j < N_; j++) L2[t * N_ + j] = sg > 0 ? row[j] / sg : 0.0;
    }
  }

 private:
  // kind 0: out [N x k] = A^T P (P [M x k]); kind 1: out [M x k] = A P (P [N x k])
  void product(int kind, const double* P, double* out) {
    if (err_) return;
    const int T = (int)(kind == 0 ? M_ : N_), O = (int)(kind == 0 ? N_ : M_);
    const dim3 grid((unsigned)((O + PBO - 1) / PBO), (unsigned)((k_ + PBC - 1) / PBC));
    if (kind == 0)
      k_panel_mfma<0><<<grid, 256, 0, s_>>>(w_.A, N_, nullptr, T, O, (int)k_, P, out);
    else
      k_panel_mfma<1><<<grid, 256, 0, s_>>>(w_.A, N_, nullptr, T, O, (int)k_, P, out);
    launch_ok();
  }
  // Cholesky-QR twice on the panel P [T x k], in place: the first pass writes P R1^-1 into the
  // scratch panel p2, the second writes (P R1^-1) R2^-1 back into P. R^-1 is applied on the
  // device; the k x k factorisations run on the host.
  void orthonormalize(double* P, int64_t T) {
    const int64_t k = k_;
    std::vector<double> G((size_t)(k * k)), R((size_t)(k * k)), Ri((size_t)(k * k));
    double* src = P;
    double* dst = w_.p2;
    for (int pass = 0; pass < 2; pass++) {
      if (err_) return;
      const dim3 grid((unsigned)((k + PBO - 1) / PBO), (unsigned)((k + PBC - 1) / PBC));
      k_panel_mfma<2><<<grid, 256, 0, s_>>>(nullptr, 0, src, (int)T, (int)k, (int)k, src, w_.G);
      launch_ok();
      note(hipMemcpyAsync(G.data(), w_.G, G.size() * 8, hipMemcpyDeviceToHost, s_));
      note(hipStreamSynchronize(s_));
      if (err_) return;
      cholesky_inverse(G, R, Ri);
      note(hipMemcpyAsync(w_.S, Ri.data(), Ri.size() * 8, hipMemcpyHostToDevice, s_));
      k_panel_times<true><<<(unsigned)((T + 63) / 64), 64, (size_t)k * 64 * 8, s_>>>(src, (int)T, (int)k, w_.S, (int)k,
                                                                                      (int)k, dst);
      launch_ok();
      std::swap(src, dst);
    }
  }
  // G + s I = R^T R (R upper), Ri = R^-1, with s = 1e-13 trace(G) / k
  void cholesky_inverse(const std::vector<double>& G, std::vector<double>& R, std::vector<double>& Ri) const {
    const int64_t k = k_;
    double tr = 0;
    for (int64_t i = 0; i < k; i++) tr += G[i * k + i];
    const double shift = 1e-13 * tr / (double)k + 1e-300;
    std::fill(R.begin(), R.end(), 0.0);
    for (int64_t j = 0; j < k; j++) {
      double d = G[j * k + j] + shift;
      for (int64_t p = 0; p < j; p++) d -= R[p * k + j] * R[p * k + j];
      const double rjj = std::sqrt(std::max(d, shift));
      R[j * k + j] = rjj;
      for (int64_t c = j + 1; c < k; c++) {
        double v = G[j * k + c];
        for (int64_t p = 0; p < j; p++) v -= R[p * k + j] * R[p * k + c];
        R[j * k + c] = v / rjj;
      }
    }
    // Ri upper triangular: R Ri = I, back substitution column by column
    std::fill(Ri.begin(), Ri.end(), 0.0);
    for (int64_t c = 0; c < k; c++) {
      for (int64_t i = c; i >= 0; i--) {
        double v = (i == c) ? 1.0 : 0.0;
        for (int64_t p = i + 1; p <= c; p++) v -= R[i * k + p] * Ri[p * k + c];
        Ri[i * k + c] = v / R[i * k + i];
      }
    }
  }
  void jacobi() {
    const int64_t k = k_;
    if (err_ || k < 2) return;
    const int64_t np = k + (k & 1);
    std::vector<int> pairs((size_t)((np - 1) * np));
    std::vector<int64_t> ring((size_t)np);
    std::iota(ring.begin(), ring.end(), 0);
    for (int64_t round = 0; round < np - 1; round++) {
      for (int64_t t = 0; t < np / 2; t++) {
        pairs[(round * (np / 2) + t) * 2] = (int)ring[t];
        pairs[(round * (np / 2) + t) * 2 + 1] = (int)ring[np - 1 - t];
      }
      const int64_t last = ring[np - 1];
      for (int64_t i = np - 1; i > 1; i--) ring[i] = ring[i - 1];
      ring[1] = last;
    }
    note(hipMemcpyAsync(w_.pairs, pairs.data(), pairs.size() * 4, hipMemcpyHostToDevice, s_));
    k_identity<<<(unsigned)((k * k + 255) / 256), 256, 0, s_>>>(w_.J, (int)k);
    launch_ok();
    for (int sweep = 0; sweep < 60 && !err_; sweep++) {
      note(hipMemsetAsync(w_.counter, 0, 4, s_));
      for (int64_t round = 0; round < np - 1; round++)
        k_jacobi_round<<<(unsigned)(np / 2), 256, 0, s_>>>(w_.Bm, N_, (int)k, w_.J, w_.pairs + round * np, 1e-13,
                                                           w_.counter);
      launch_ok();
      int rotated = 0;
      note(hipMemcpyAsync(&rotated, w_.counter, 4, hipMemcpyDeviceToHost, s_));
      note(hipStreamSynchronize(s_));
      if (rotated == 0) break;
    }
  }
  void launch_ok() { note(hipGetLastError()); }
  void note(hipError_t e) {
    if (err_ == hipSuccess && e != hipSuccess) err_ = e;
  }
  int64_t M_, N_, k_, r_;
  hipStream_t s_;
  SvdWorkspace w_{};
  hipError_t err_ = hipSuccess;
};

}  // namespace dev

int64_t device_svd_columns(int64_t M, int64_t N, int64_t r) {
  const int64_t k = host::randomized_panel_columns(M, N, r);
  return k <= kMaxDeviceK ? k : 0;
}

size_t device_svd_bytes(int64_t M, int64_t N, int64_t k, int64_t r) {
  return (size_t)dev::SvdWorkspace::layout(M, N, k, r, nullptr, nullptr);
}

int run_split_on_device(const float* A, int64_t M, int64_t N, int64_t r, void* workspace, void* stream, double* L1,
                        double* L2) {
  const int64_t k = device_svd_columns(M, N, r);
  if (k == 0) {
    host::truncated_svd(A, M, N, N, r, L1, L2);
    return 0;
  }
  dev::DeviceSvd svd(A, M, N, k, r, reinterpret_cast<uint8_t*>(workspace), (hipStream_t)stream);
  svd.run(16, L1, L2);
  hipError_t e = svd.error();
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  return (int)e;
}

}  // namespace svdq
