// Blocked right-looking Cholesky Sigma = U^T U in fp64 (WaterSIC page, Sommario tecnico §2
// item 1 factorizes the activation covariance; U here is the transpose of the page's L).
//
// Per 64-column step kb (driven from the host):
//   k_potrf_panel : the block row [kb, kb+64) x [kb, n). Workgroup b > 0 owns a 64-column slab
//                   of it; every workgroup factors the 64 x 64 diagonal block itself (the same
//                   instructions on the same data, so every copy of U_kk is bitwise identical)
//                   and applies each pivot's elimination to its slab as it goes, which is the
//                   triangular solve X = U_kk^-T A_k,rest. Thread (wave w, lane j) holds rows
//                   16w .. 16w+15 of column j of the diagonal block and of its slab. At pivot k
//                   the owning wave publishes row k of both through LDS; every thread reads the
//                   pivot and the 16 row entries it needs with all loads in flight and scales
//                   by 1/sqrt(p). The update has no branches (rows above the pivot meet a zero
//                   multiplier); the pivot row buffers alternate with the parity of k, so one
//                   barrier per pivot suffices. Nothing is written to global memory inside the
//                   pivot loop.
//   trailing      : A_rest,rest -= X^T X on upper tiles (fp64 MFMA GEMM, k-major operands)
// The first failing pivot (1-based, global) is recorded in *info; later steps see it and
// return immediately.
#include "common.h"

namespace wsic {
namespace {

constexpr int NB = 64;
constexpr int RPW = NB / 4;  // rows per wave

// 1/sqrt(p) to ~1 ulp: hardware estimate refined by two Newton steps
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
  const double h = 0.5 * p;
  y = y * fma(-h * y, y, 1.5);
  y = y * fma(-h * y, y, 1.5);
  return y;
}

__global__ __launch_bounds__(256) void k_potrf_panel(double* A, int64_t lda, int64_t kb, int nbk,
                                                     int64_t n, int64_t* info) {
  // raw row k of the diagonal block and of this workgroup's slab, double-buffered by the parity
  // of k so that one barrier per pivot separates its writes from the previous pivot's reads
  __shared__ double row[2][NB];
  __shared__ double srow[2][NB];
  if (*info != 0) return;
  const int j = threadIdx.x & 63;
  // the wave index, known to the compiler as wave-uniform
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int64_t c = kb + (int64_t)b * NB + j;  // slab column (b > 0)
  const bool has_slab = b > 0;
  const bool cin = has_slab && c < n;

  double a[RPW], sl[RPW];  // rows 16 w + s of column j: diagonal block, slab
#pragma unroll
  for (int s = 0; s < RPW; ++s) {
    const int i = RPW * w + s;
    a[s] = (i <= j && j < nbk) ? A[(kb + i) * lda + kb + j] : (i == j ? 1.0 : 0.0);
    sl[s] = (cin && i < nbk) ? A[(kb + i) * lda + c] : 0.0;
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (k < nbk) {  // uniform
      const int wk = k / RPW, sk = k % RPW, pb = k & 1;
      if (w == wk) {
        // row k of the block is published with zeros left of the diagonal (the lower-triangle
        // entries a thread holds are scratch, never stored)
        row[pb][j] = (j >= k) ? a[sk] : 0.0;
        srow[pb][j] = sl[sk];
      }
      __syncthreads();
      const double p = row[pb][k];
      const double rj = row[pb][j];
      const double xs = srow[pb][j];
      if (!(p > 0.0) || !isfinite(p)) {  // uniform: every thread sees the same pivot
        if (b == 0 && threadIdx.x == 0) *info = kb + k + 1;
        return;
      }
      const double inv = rsqrt_f64(p);
      const double sj = rj * inv;  // U(k, j)
      const double xk = xs * inv;  // X(k, c)
      // Branch-free elimination: the published row k is zero left of the diagonal, so rows above
      // the pivot get a zero multiplier and keep their values, and no upper entry is touched by
      // a column left of the pivot; the pivot row itself is then overwritten with its scaled
      // entries.
      double rr[RPW];
#pragma unroll
      for (int s = 0; s < RPW; ++s) rr[s] = row[pb][RPW * w + s];
#pragma unroll
      for (int s = 0; s < RPW; ++s) {
        const double uki = rr[s] * inv;  // U(k, i) for i > k
        a[s] = fma(-uki, sj, a[s]);
        sl[s] = fma(-uki, xk, sl[s]);
      }
      const bool own = (w == wk);
      a[sk] = own ? ((j == k) ? p * inv : sj) : a[sk];
      sl[sk] = own ? xk : sl[sk];
    }
  }
#pragma unroll
  for (int s = 0; s < RPW; ++s) {
    const int i = RPW * w + s;
    if (i < nbk) {
      if (b == 0) {
        if (j < nbk) A[(kb + i) * lda + kb + j] = (i <= j) ? a[s] : 0.0;
      } else if (cin) {
        A[(kb + i) * lda + c] = sl[s];
      }
    }
  }
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

int launch_potrf_panel(double* A, int64_t lda, int64_t kb, int nbk, int64_t n, int64_t* info,
                       hipStream_t st) {
  if (nbk <= 0 || nbk > NB) {
    set_error("internal: potrf block %d", nbk);
    return WSIC_E_INVAL;
  }
  const int64_t m = n - kb - nbk;  // columns right of the diagonal block
  const unsigned blocks = 1 + (unsigned)((m + NB - 1) / NB);
  const double work = (double)nbk * nbk * nbk / 3.0 + (double)nbk * nbk * m;
  WSIC_LAUNCH("potrf_panel", work, st, k_potrf_panel, dim3(blocks), dim3(256), 0, A, lda, kb, nbk, n,
              info);
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
