// Truncated SVD for the one-time weight preparation (host, float64, OpenMP).
//
// Used by split_weight: the best rank-r approximation of the smoothed weight, as the
// exercise page "SVDQuant Smoothing, Low-rank and Residual Quantization" defines it
// ("Formula and conventions" item 2: left @ right is a best rank-r approximation from a
// truncated SVD; any equivalent factorisation is accepted).
//
// Two routes, no LAPACK:
//  * small matrices (min(M,N) <= 512, or rank + oversampling >= min(M,N)): one-sided
//    (Hestenes) Jacobi on the whole matrix — a full SVD, exact up to rounding, so rank 0
//    and full rank behave exactly;
//  * large matrices: randomized subspace iteration (Halko, Martinsson & Tropp 2011,
//    Algorithm 4.4) with k = rank + 32 columns and 16 power iterations (enough for the
//    rank-r Frobenius error to sit within ~1e-4 of the Eckart-Young optimum on noise-bulk spectra),
//    then a Rayleigh-Ritz step (one-sided Jacobi on the k x N projection Q^T A).
//
// Every parallel loop writes disjoint outputs and sums in a fixed order, so results do not
// depend on the thread count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <vector>

#include <omp.h>

#include "host_svd.h"

namespace svdq {
namespace host {

namespace {

typedef double v4d __attribute__((vector_size(32)));

constexpr int MR = 6, NR = 8;
constexpr int64_t KC = 256, MC = 96, NC = 2048, NSUB = 256;

inline v4d load4(const double* p) {
  v4d v;
  std::memcpy(&v, p, sizeof(v));
  return v;
}
inline void store4(double* p, v4d v) { std::memcpy(p, &v, sizeof(v)); }

// C[MR x NR] (+)= Ap[kc x MR] (p-major) * Bp[kc x NR] (p-major); edges masked by mr, nr.
void micro_kernel(int64_t kc, const double* Ap, const double* Bp, double* C, int64_t ldc, int mr, int nr,
                  bool accumulate) {
  v4d c[MR][2];
  for (int i = 0; i < MR; i++) c[i][0] = c[i][1] = v4d{0, 0, 0, 0};
  for (int64_t p = 0; p < kc; p++) {
    const v4d b0 = load4(Bp + p * NR), b1 = load4(Bp + p * NR + 4);
    for (int i = 0; i < MR; i++) {
      const double a = Ap[p * MR + i];
      const v4d av = {a, a, a, a};
      c[i][0] += av * b0;
      c[i][1] += av * b1;
    }
  }
  for (int i = 0; i < mr; i++) {
    double tmp[NR];
    store4(tmp, c[i][0]);
    store4(tmp + 4, c[i][1]);
    double* crow = C + i * ldc;
    for (int j = 0; j < nr; j++) crow[j] = accumulate ? crow[j] + tmp[j] : tmp[j];
  }
}

template <class TA>
void pack_a(int64_t mc, int64_t kc, const TA* A, int64_t ars, int64_t acs, double* Ap) {
  for (int64_t ir = 0; ir < mc; ir += MR) {
    const int mr = (int)std::min<int64_t>(MR, mc - ir);
    double* dst = Ap + ir * kc;
    for (int64_t p = 0; p < kc; p++)
      for (int i = 0; i < MR; i++) dst[p * MR + i] = i < mr ? (double)A[(ir + i) * ars + p * acs] : 0.0;
  }
}

template <class TB>
void pack_b(int64_t kc, int64_t nc, const TB* B, int64_t brs, int64_t bcs, double* Bp) {
  const int64_t panels = (nc + NR - 1) / NR;
#pragma omp parallel for schedule(static)
  for (int64_t jp = 0; jp < panels; jp++) {
    const int64_t j0 = jp * NR;
    const int nr = (int)std::min<int64_t>(NR, nc - j0);
    double* dst = Bp + j0 * kc;
    if (bcs == 1) {
      for (int64_t p = 0; p < kc; p++)
        for (int j = 0; j < NR; j++) dst[p * NR + j] = j < nr ? (double)B[p * brs + j0 + j] : 0.0;
    } else {
      for (int j = 0; j < NR; j++)
        for (int64_t p = 0; p < kc; p++) dst[p * NR + j] = j < nr ? (double)B[p * brs + (j0 + j) * bcs] : 0.0;
    }
  }
}

}  // namespace

template <class TA, class TB>
void gemm(int64_t M, int64_t N, int64_t K, const TA* A, int64_t ars, int64_t acs, const TB* B, int64_t brs,
          int64_t bcs, double* C, int64_t ldc) {
  if (M <= 0 || N <= 0) return;
  if (K <= 0) {
    for (int64_t i = 0; i < M; i++) std::fill(C + i * ldc, C + i * ldc + N, 0.0);
    return;
  }
  std::vector<double> Bp((size_t)KC * (NC + NR));
  for (int64_t jc = 0; jc < N; jc += NC) {
    const int64_t nc = std::min(NC, N - jc);
    for (int64_t pc = 0; pc < K; pc += KC) {
      const int64_t kc = std::min(KC, K - pc);
      pack_b(kc, nc, B + pc * brs + jc * bcs, brs, bcs, Bp.data());
      const int64_t mblocks = (M + MC - 1) / MC, nblocks = (nc + NSUB - 1) / NSUB;
#pragma omp parallel
      {
        std::vector<double> Ap((size_t)(MC + MR) * KC);
#pragma omp for collapse(2) schedule(dynamic)
        for (int64_t ib = 0; ib < mblocks; ib++) {
          for (int64_t jb = 0; jb < nblocks; jb++) {
            const int64_t ic = ib * MC, mc = std::min(MC, M - ic);
            pack_a(mc, kc, A + ic * ars + pc * acs, ars, acs, Ap.data());
            const int64_t j_lo = jb * NSUB, j_hi = std::min(nc, j_lo + NSUB);
            for (int64_t jr = j_lo; jr < j_hi; jr += NR) {
              const int nr = (int)std::min<int64_t>(NR, j_hi - jr);
              for (int64_t ir = 0; ir < mc; ir += MR) {
                const int mr = (int)std::min<int64_t>(MR, mc - ir);
                micro_kernel(kc, Ap.data() + ir * kc, Bp.data() + jr * kc, C + (ic + ir) * ldc + jc + jr, ldc, mr,
                             nr, pc > 0);
              }
            }
          }
        }
      }
    }
  }
}

template void gemm<double, double>(int64_t, int64_t, int64_t, const double*, int64_t, int64_t, const double*,
                                   int64_t, int64_t, double*, int64_t);
template void gemm<double, float>(int64_t, int64_t, int64_t, const double*, int64_t, int64_t, const float*,
                                  int64_t, int64_t, double*, int64_t);
template void gemm<float, double>(int64_t, int64_t, int64_t, const float*, int64_t, int64_t, const double*,
                                  int64_t, int64_t, double*, int64_t);
template void gemm<float, float>(int64_t, int64_t, int64_t, const float*, int64_t, int64_t, const float*, int64_t,
                                 int64_t, double*, int64_t);

namespace {

double dot(const double* a, const double* b, int64_t n) {
  double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  int64_t i = 0;
  for (; i + 4 <= n; i += 4) {
    s0 += a[i] * b[i];
    s1 += a[i + 1] * b[i + 1];
    s2 += a[i + 2] * b[i + 2];
    s3 += a[i + 3] * b[i + 3];
  }
  for (; i < n; i++) s0 += a[i] * b[i];
  return (s0 + s1) + (s2 + s3);
}

inline void rotate(double* x, double* y, int64_t n, double c, double s) {
  for (int64_t i = 0; i < n; i++) {
    const double xi = x[i], yi = y[i];
    x[i] = c * xi - s * yi;
    y[i] = s * xi + c * yi;
  }
}

// Deterministic standard normals: splitmix64 + Box-Muller.
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

// Orthonormalise the k columns (length m, column c at Q + c*m) by classical Gram-Schmidt
// applied twice; a column that vanishes is replaced by a fresh pseudo-random direction.
void orthonormalize(double* Q, int64_t m, int64_t k, uint64_t seed) {
  Normal rng(seed);
  std::vector<double> h((size_t)k);
  for (int64_t j = 0; j < k; j++) {
    double* v = Q + j * m;
    for (int attempt = 0; attempt < 4; attempt++) {
      const double n0 = std::sqrt(dot(v, v, m));
      for (int pass = 0; pass < 2; pass++) {
#pragma omp parallel for schedule(static) if (m * j > 65536)
        for (int64_t c = 0; c < j; c++) h[c] = dot(Q + c * m, v, m);
        const int64_t chunk = 512, nchunks = (m + chunk - 1) / chunk;
#pragma omp parallel for schedule(static) if (m * j > 65536)
        for (int64_t ch = 0; ch < nchunks; ch++) {
          const int64_t i0 = ch * chunk, i1 = std::min(m, i0 + chunk);
          for (int64_t c = 0; c < j; c++) {
            const double hc = h[c];
            const double* qc = Q + c * m;
            for (int64_t i = i0; i < i1; i++) v[i] -= qc[i] * hc;
          }
        }
      }
      const double n1 = std::sqrt(dot(v, v, m));
      if (n1 > 1e-10 * n0 && n1 > 0) {
        for (int64_t i = 0; i < m; i++) v[i] /= n1;
        break;
      }
      for (int64_t i = 0; i < m; i++) v[i] = rng();  // dependent column: restart from noise
      if (attempt == 3) std::fill(v, v + m, 0.0);
    }
  }
}

}  // namespace

void jacobi_columns(double* G, int64_t m, int64_t n, int64_t ldg, double* V, int64_t ldv) {
  for (int64_t c = 0; c < n; c++)
    for (int64_t i = 0; i < n; i++) V[c * ldv + i] = (i == c) ? 1.0 : 0.0;
  if (n < 2) return;
  const int64_t np = n + (n & 1);  // round-robin over an even count (index n is a bye)
  std::vector<int64_t> ring((size_t)np);
  std::iota(ring.begin(), ring.end(), 0);
  const double tol = 1e-13;  // relative orthogonality at which a pair counts as converged
  for (int sweep = 0; sweep < 60; sweep++) {
    int64_t rotated = 0;
    for (int64_t round = 0; round < np - 1; round++) {
#pragma omp parallel for schedule(dynamic) reduction(+ : rotated) if (m * n > 200000)
      for (int64_t t = 0; t < np / 2; t++) {
        int64_t p = ring[t], q = ring[np - 1 - t];
        if (p >= n || q >= n) continue;
        if (p > q) std::swap(p, q);
        double* gp = G + p * ldg;
        double* gq = G + q * ldg;
        const double alpha = dot(gp, gp, m), beta = dot(gq, gq, m), gamma = dot(gp, gq, m);
        if (!(std::fabs(gamma) > tol * std::sqrt(alpha * beta))) continue;
        const double zeta = (beta - alpha) / (2.0 * gamma);
        const double t_ = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::hypot(1.0, zeta));
        const double c = 1.0 / std::sqrt(1.0 + t_ * t_), s = c * t_;
        rotate(gp, gq, m, c, s);
        rotate(V + p * ldv, V + q * ldv, n, c, s);
        rotated++;
      }
      // rotate the ring, keeping position 0 fixed
      const int64_t last = ring[np - 1];
      for (int64_t i = np - 1; i > 1; i--) ring[i] = ring[i - 1];
      ring[1] = last;
    }
    if (rotated == 0) break;
  }
}

namespace {

// Column order by decreasing norm (ties by index, so the order is deterministic).
std::vector<int64_t> order_by_norm(const double* G, int64_t m, int64_t n, int64_t ldg, std::vector<double>& sigma) {
  sigma.assign((size_t)n, 0.0);
  for (int64_t c = 0; c < n; c++) sigma[c] = std::sqrt(dot(G + c * ldg, G + c * ldg, m));
  std::vector<int64_t> ord((size_t)n);
  std::iota(ord.begin(), ord.end(), 0);
  std::stable_sort(ord.begin(), ord.end(), [&](int64_t a, int64_t b) { return sigma[a] > sigma[b]; });
  return ord;
}

void full_svd(const float* A, int64_t M, int64_t N, int64_t lda, int64_t r, double* L1, double* L2) {
  std::vector<double> sigma;
  if (N <= M) {
    // columns of A: A J = W, A = W J^T  ->  L1 = W_r, L2 = J_r^T
    std::vector<double> G((size_t)M * N), V((size_t)N * N);
    for (int64_t i = 0; i < M; i++)
      for (int64_t j = 0; j < N; j++) G[j * M + i] = A[i * lda + j];
    jacobi_columns(G.data(), M, N, M, V.data(), N);
    auto ord = order_by_norm(G.data(), M, N, M, sigma);
    for (int64_t t = 0; t < r; t++) {
      const int64_t c = ord[t];
      for (int64_t i = 0; i < M; i++) L1[i * r + t] = G[c * M + i];
      for (int64_t j = 0; j < N; j++) L2[t * N + j] = V[c * N + j];
    }
  } else {
    // rows of A: A^T J = W, A = J W^T  ->  L1 = J_r diag(sigma_r), L2 = (W_r / sigma_r)^T
    std::vector<double> G((size_t)N * M), V((size_t)M * M);
    for (int64_t i = 0; i < M; i++)
      for (int64_t j = 0; j < N; j++) G[i * N + j] = A[i * lda + j];
    jacobi_columns(G.data(), N, M, N, V.data(), M);
    auto ord = order_by_norm(G.data(), N, M, N, sigma);
    for (int64_t t = 0; t < r; t++) {
      const int64_t c = ord[t];
      const double s = sigma[c];
      for (int64_t i = 0; i < M; i++) L1[i * r + t] = s * V[c * M + i];
      for (int64_t j = 0; j < N; j++) L2[t * N + j] = s > 0 ? G[c * N + j] / s : 0.0;
    }
  }
}

void randomized_svd(const float* A, int64_t M, int64_t N, int64_t lda, int64_t r, int64_t k, int power_iters,
                    double* L1, double* L2) {
  // the large products with A
  auto prod = [&](int kind, const double* P, double* C) {
    if (kind == 0)
      gemm<double, float>(k, N, M, P, M, 1, A, lda, 1, C, N);  // C^T [k x N] = P^T [k x M] * A [M x N]
    else
      gemm<double, float>(k, M, N, P, N, 1, A, 1, lda, C, M);  // C^T [k x M] = P^T [k x N] * A^T [N x M]
  };
  // Panels are stored column-major: column c of a [rows x k] panel at P + c*rows.
  std::vector<double> Om((size_t)N * k), Q((size_t)M * k), Z((size_t)N * k);
  Normal rng(0x5EEDull + (uint64_t)M * 1000003ull + (uint64_t)N);
  for (auto& v : Om) v = rng();
  prod(1, Om.data(), Q.data());  // Y = A * Om
  orthonormalize(Q.data(), M, k, 11);
  for (int it = 0; it < power_iters; it++) {
    prod(0, Q.data(), Z.data());  // Z = A^T Q
    orthonormalize(Z.data(), N, k, 101 + it);
    prod(1, Z.data(), Q.data());  // Q = A Z
    orthonormalize(Q.data(), M, k, 1001 + it);
  }
  // Rayleigh-Ritz: Bs = Q^T A [k x N] (row l = column l of Bs^T), Bs^T J = W.
  std::vector<double> Bs((size_t)k * N), J((size_t)k * k);
  prod(0, Q.data(), Bs.data());
  jacobi_columns(Bs.data(), N, k, N, J.data(), k);
  std::vector<double> sigma;
  auto ord = order_by_norm(Bs.data(), N, k, N, sigma);
  // A ~= (Q J) W^T:  L1 = (Q J)_r diag(sigma_r),  L2 = (W_r / sigma_r)^T
  std::vector<double> Jr((size_t)k * r);
  for (int64_t t = 0; t < r; t++)
    for (int64_t p = 0; p < k; p++) Jr[p * r + t] = J[ord[t] * k + p];
  gemm<double, double>(M, r, k, Q.data(), 1, M, Jr.data(), r, 1, L1, r);
  for (int64_t t = 0; t < r; t++) {
    const double s = sigma[ord[t]];
    for (int64_t i = 0; i < M; i++) L1[i * r + t] *= s;
    const double* w = Bs.data() + ord[t] * N;
    for (int64_t j = 0; j < N; j++) L2[t * N + j] = s > 0 ? w[j] / s : 0.0;
  }
}

}  // namespace

int64_t randomized_panel_columns(int64_t M, int64_t N, int64_t r) {
  const int64_t n = std::min(M, N);
  const int64_t k = std::min(n, r + 32);
  return (r <= 0 || n <= 512 || k >= n) ? 0 : k;
}

void truncated_svd(const float* A, int64_t M, int64_t N, int64_t lda, int64_t r, double* L1, double* L2) {
  if (r <= 0) return;
  const int64_t k = randomized_panel_columns(M, N, r);
  if (k == 0)
    full_svd(A, M, N, lda, r, L1, L2);
  else
    randomized_svd(A, M, N, lda, r, k, 16, L1, L2);
}

}  // namespace host
}  // namespace svdq
