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
  // pivots in four groups of RPW: the group loop stays a loop (code size: the instruction cache
  // holds one group), the RPW pivots of a group are unrolled so register indices are constants
#pragma unroll 1
  for (int wk = 0; wk < NB / RPW; ++wk) {
#pragma unroll
  for (int sk = 0; sk < RPW; ++sk) {
    const int k = RPW * wk + sk;
    if (k < nbk) {  // uniform
      const int pb = sk & 1;
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
      // entries. U(k,i) U(k,j) = row_k(i) * (U(k,j) / sqrt(p)): one multiplier per column.
      const double mj = sj * inv, mx = xk * inv;
      double rr[RPW];
#pragma unroll
      for (int s = 0; s < RPW; ++s) rr[s] = row[pb][RPW * w + s];
#pragma unroll
      for (int s = 0; s < RPW; ++s) {
        a[s] = fma(-rr[s], mj, a[s]);
        sl[s] = fma(-rr[s], mx, sl[s]);
      }
      const bool own = (w == wk);
      a[sk] = own ? ((j == k) ? p * inv : sj) : a[sk];
      sl[sk] = own ? xk : sl[sk];
    }
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

// Trailing update A22 -= X^T X after a block row: X = rows r0 .. r0+KR-1 of A at columns
// c0 .. c0+m-1 (the solved block row), A22 = A[c0.., c0..] (m x m), upper tiles only.
// One 256-thread workgroup per 64 x 64 upper tile (tiles enumerated triangularly): the C tile is
// loaded into registers first, then the KR x 64 column strips of X for the tile's rows and
// columns go global -> LDS directly (global_load_lds_dwordx4, lane l of an instruction at byte
// 16 l) in their natural layout, [k][col], which is already the conflict-free layout of the
// v_mfma_f64_16x16x4 operands (16 lanes read 16 consecutive doubles of one k row). Diagonal
// tiles load one strip. 4 waves in 2 x 2, each 32 x 32 = 2 x 2 fragments.
// Requirements (checked by the launcher): A 16-byte aligned, lda even, c0 even.
namespace cupd {
constexpr int T = 64;
typedef __attribute__((address_space(3))) void lds_void;
typedef double d4 __attribute__((ext_vector_type(4)));
}  // namespace cupd

template <int KR>
__global__ __launch_bounds__(256) void k_chol_update(double* A, int64_t lda, int64_t r0, int64_t c0,
                                                     int64_t m, const int64_t* info) {
  using namespace cupd;
  __shared__ __attribute__((aligned(1024))) double Xs[2][KR][T];
  if (*info != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // triangular tile index: bid -> (tm <= tn)
  const int64_t bid = blockIdx.x;
  int64_t tn = (int64_t)((sqrt(8.0 * (double)bid + 1.0) - 1.0) * 0.5);
  while ((tn + 1) * (tn + 2) / 2 <= bid) ++tn;
  while (tn * (tn + 1) / 2 > bid) --tn;
  const int64_t tm = bid - tn * (tn + 1) / 2;
  const int64_t i0 = tm * T, j0 = tn * T;
  const bool diag = (tm == tn);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lk = lane >> 4;

  // C tile of this lane (result layout), loaded first
  double cold[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t ii = i0 + wm * 32 + i * 16 + lk + 4 * r;
        const int64_t jj = j0 + wn * 32 + j * 16 + lr;
        cold[i][j][r] = (ii < m && jj < m) ? A[(c0 + ii) * lda + c0 + jj] : 0.0;
      }

  // strips: KR rows x 64 columns = KR * 32 chunks of 16 bytes, KR / 2 instructions per strip
  constexpr int INS = KR / 2 / 4;  // per wave per strip
  const int64_t clast = (m - 1) & ~(int64_t)1;  // last chunk start inside the row
#pragma unroll
  for (int sidx = 0; sidx < 2; ++sidx) {
    if (sidx == 1 && diag) break;  // uniform
    const int64_t col0 = (sidx == 0) ? i0 : j0;
#pragma unroll
    for (int h = 0; h < INS; ++h) {
      const int ins = INS * wave + h;
      const int p = 64 * ins + lane;
      const int t = p >> 5, ch = p & 31;
      int64_t cc = col0 + 2 * ch;
      cc = cc < clast ? cc : clast;
      __builtin_amdgcn_global_load_lds((const void*)(A + (r0 + t) * lda + c0 + cc),
                                       (lds_void*)(&Xs[sidx][0][0] + 128 * ins), 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const double(*Xa)[T] = Xs[0];
  const double(*Xb)[T] = diag ? Xs[0] : Xs[1];
  d4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (d4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k4 = 0; k4 < KR / 4; ++k4) {
    const int k = 4 * k4 + lk;
    double a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = Xa[k][wm * 32 + i * 16 + lr];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = Xb[k][wn * 32 + j * 16 + lr];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t ii = i0 + wm * 32 + i * 16 + lk + 4 * r;
        const int64_t jj = j0 + wn * 32 + j * 16 + lr;
        if (ii < m && jj < m) A[(c0 + ii) * lda + c0 + jj] = cold[i][j][r] - acc[i][j][r];
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

bool chol_update_ok(const double* A, int64_t lda, int64_t c0, int kr) {
  return kr == NB && (((uintptr_t)A) & 15) == 0 && (lda % 2) == 0 && (c0 % 2) == 0;
}

int launch_chol_update(double* A, int64_t lda, int64_t r0, int64_t c0, int64_t m, int kr,
                       const int64_t* info, hipStream_t st) {
  if (m <= 0) return WSIC_OK;
  if (!chol_update_ok(A, lda, c0, kr)) {
    set_error("internal: chol update preconditions");
    return WSIC_E_INVAL;
  }
  const int64_t t = (m + cupd::T - 1) / cupd::T;
  const int64_t tiles = t * (t + 1) / 2;
  const double work = (double)m * (double)(m + 1) * (double)kr;
  WSIC_LAUNCH("chol_update", work, st, k_chol_update<NB>, dim3((unsigned)tiles), dim3(256), 0, A,
              lda, r0, c0, m, info);
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
