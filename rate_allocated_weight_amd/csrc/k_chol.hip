// Blocked right-looking Cholesky Sigma = U^T U in fp64 (WaterSIC page, Sommario tecnico §2
// item 1 factorizes the activation covariance; U here is the transpose of the page's L).
//
// Per 64-column step kb (driven from the host):
//   k_potrf_diag : one workgroup factors the 64 x 64 diagonal block in LDS
//   k_trsm_row   : the block row to its right, X = U_kk^-T A_k,rest, one thread per column
//   trailing     : A_rest,rest -= X^T X on upper tiles (fp64 MFMA GEMM, k-major operands)
// The first failing pivot (1-based, global) is recorded in *info; later steps see it and
// return immediately, so a failed factorization costs no more launches' worth of work.
#include "common.h"

namespace wsic {
namespace {

constexpr int NB = 64;

__global__ __launch_bounds__(256) void k_potrf_diag(double* A, int64_t lda, int64_t kb, int nbk,
                                                    int64_t* info) {
  __shared__ double a[NB][NB + 1];
  __shared__ int fail;
  if (*info != 0) return;
  const int tid = threadIdx.x;
  // thread (ty, tx): column tx of the block, rows ty, ty+4, ... (all 16 loads in flight)
  const int tx = tid & 63, ty = tid >> 6;
  {
    double v[NB / 4];
#pragma unroll
    for (int s = 0; s < NB / 4; ++s) {
      const int i = ty + 4 * s;
      v[s] = (i < nbk && tx < nbk && tx >= i) ? A[(kb + i) * lda + kb + tx] : 0.0;
    }
#pragma unroll
    for (int s = 0; s < NB / 4; ++s) a[ty + 4 * s][tx] = v[s];
  }
  (void)fail;
  for (int k = 0; k < nbk; ++k) {
    __syncthreads();
    const double p = a[k][k];  // every thread sees the same pivot: uniform exit
    if (!(p > 0.0) || !isfinite(p)) {
      if (tid == 0) *info = kb + k + 1;
      return;
    }
    const double d = sqrt(p);
    __syncthreads();  // pivot read by all before row k changes
    if (ty == 0 && tx >= k && tx < nbk) a[k][tx] = (tx == k) ? d : a[k][tx] / d;
    __syncthreads();
    if (tx > k && tx < nbk) {
      // all 32 LDS reads issued before any FMA (rows ty + 4s are in bounds of the tile)
      const double akj = a[k][tx];
      double av[NB / 4], ak[NB / 4];
#pragma unroll
      for (int s = 0; s < NB / 4; ++s) {
        av[s] = a[ty + 4 * s][tx];
        ak[s] = a[k][ty + 4 * s];
      }
#pragma unroll
      for (int s = 0; s < NB / 4; ++s) {
        const int i = ty + 4 * s;
        if (i > k && i <= tx) a[i][tx] = fma(-ak[s], akj, av[s]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) {
    const int i = ty + 4 * s;
    if (i < nbk && tx < nbk) A[(kb + i) * lda + kb + tx] = (tx >= i) ? a[i][tx] : 0.0;
  }
}

constexpr int TRSM_THREADS = 64;

__global__ __launch_bounds__(TRSM_THREADS) void k_trsm_row(double* A, int64_t lda, int64_t kb,
                                                           int64_t n, const int64_t* info) {
  __shared__ __attribute__((aligned(16))) double u[NB][NB];  // U_kk, row-major
  if (*info != 0) return;
  const int tid = threadIdx.x;
  // thread tid fills column tid of U_kk: 64 loads in flight, then the LDS stores
  {
    double v[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) v[t] = (tid >= t) ? A[(kb + t) * lda + kb + tid] : 0.0;
#pragma unroll
    for (int t = 0; t < NB; ++t) u[t][tid] = v[t];
  }
  __syncthreads();
  const int64_t c = kb + NB + (int64_t)blockIdx.x * TRSM_THREADS + tid;
  if (c >= n) return;
  double x[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) x[t] = A[(kb + t) * lda + c];
  // U_kk^T x' = x  (U_kk^T lower): forward substitution, column-oriented so that the updates
  // of different rows are independent (x_s still accumulates its terms in increasing t)
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    x[t] = x[t] / u[t][t];
#pragma unroll
    for (int s = t + 1; s < NB; ++s) x[s] = fma(-u[t][s], x[t], x[s]);
  }
#pragma unroll
  for (int t = 0; t < NB; ++t) A[(kb + t) * lda + c] = x[t];
}

__global__ void k_zero_lower(double* A, int64_t n, int64_t lda) {
  const int64_t total = n * n;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / n, j = e % n;
    if (i > j) A[i * lda + j] = 0.0;
  }
}

}  // namespace

int launch_potrf_diag(double* A, int64_t lda, int64_t kb, int nbk, int64_t* info, hipStream_t st) {
  if (nbk <= 0 || nbk > NB) {
    set_error("internal: potrf block %d", nbk);
    return WSIC_E_INVAL;
  }
  WSIC_LAUNCH("potrf_diag", (double)nbk * nbk * nbk / 3.0, st, k_potrf_diag, dim3(1), dim3(256), 0,
              A, lda, kb, nbk, info);
  return WSIC_OK;
}

int launch_trsm_row(double* A, int64_t lda, int64_t kb, int nbk, int64_t n, const int64_t* info,
                    hipStream_t st) {
  if (nbk != NB) {
    set_error("internal: trsm block %d", nbk);
    return WSIC_E_INVAL;
  }
  const int64_t m = n - kb - NB;
  if (m <= 0) return WSIC_OK;
  WSIC_LAUNCH("trsm_row", (double)NB * NB * m, st, k_trsm_row,
              dim3((unsigned)((m + TRSM_THREADS - 1) / TRSM_THREADS)), dim3(TRSM_THREADS), 0, A, lda,
              kb, n, info);
  return WSIC_OK;
}

int launch_zero_lower(double* A, int64_t n, int64_t lda, hipStream_t st) {
  int64_t blocks = (n * n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  WSIC_LAUNCH("zero_lower", 4.0 * (double)n * n, st, k_zero_lower, dim3((unsigned)blocks), dim3(256),
              0, A, n, lda);
  return WSIC_OK;
}

}  // namespace wsic
