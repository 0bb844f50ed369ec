// Host linear algebra for the one-time weight preparation (float64, OpenMP).
#pragma once
#include <cstdint>

namespace svdq {
namespace host {

// C[M x N] = op(A)[M x K] * op(B)[K x N], overwriting C (row-major, row stride ldc).
// Element (i, p) of op(A) is A[i*ars + p*acs]; element (p, j) of op(B) is B[p*brs + j*bcs].
template <class TA, class TB>
void gemm(int64_t M, int64_t N, int64_t K, const TA* A, int64_t ars, int64_t acs, const TB* B, int64_t brs,
          int64_t bcs, double* C, int64_t ldc);

// One-sided Jacobi: rotates the n columns of G (length m, column c at G + c*ldg) until they
// are mutually orthogonal; V (n x n, column c at V + c*ldv) receives the product of the
// rotations, so that G_out = G_in * V.
void jacobi_columns(double* G, int64_t m, int64_t n, int64_t ldg, double* V, int64_t ldv);

// Rank-r truncated SVD of A [M x N] (row stride lda): L1 [M x r] = U_r diag(sigma_r),
// L2 [r x N] = V_r^T, both row-major contiguous, sigma descending.
void truncated_svd(const float* A, int64_t M, int64_t N, int64_t lda, int64_t r, double* L1, double* L2);

// Columns of the randomized route's panels for rank r of an M x N matrix (0: the full
// Jacobi route is used and no panel products are needed).
int64_t randomized_panel_columns(int64_t M, int64_t N, int64_t r);

}  // namespace host
}  // namespace svdq
