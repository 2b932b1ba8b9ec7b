// Blocked right-looking Cholesky Sigma = U^T U in fp64 (WaterSIC page, Sommario tecnico §2
// item 1 factorizes the activation covariance; U here is the transpose of the page's L).
//
// Per 64-column step kb (driven from the host):
//   k_potrf_panel : the block row [kb, kb+64) x [kb, n). Workgroup b > 0 owns a 64-column slab
//                   of it; every workgroup factors the 64 x 64 diagonal block itself (the same
//                   instructions on the same data, so every copy of U_kk is bitwise identical)
//                   and applies each pivot's elimination to its slab as it goes, which is the
//                   triangular solve X = U_kk^-T A_k,rest. Thread (wave w, lane j) holds rows
//                   8w .. 8w+7 of column j of the diagonal block and of its slab. Pivots go in
//                   groups of 8: wave w factors pivots 8w .. 8w+7 on its own rows (pivot and
//                   row entries by readlane, no workgroup barrier), publishes those 8 rows of U
//                   and X through LDS, and after one barrier the waves below apply them as one
//                   rank-8 update. Nothing is written to global memory inside the pivot loop.
//   trailing      : A_rest,rest -= X^T X on upper tiles (fp64 MFMA GEMM, k-major operands).
//                   k_chol_step launches it together with the next panel, whose workgroups
//                   first apply the update to the next block row themselves.
// A panel's factored diagonal block goes to one of two NB x NB slots and reaches A in the next
// launch (or a final copy): with more panel workgroups than fit on the chip at once, a late
// workgroup would otherwise read workgroup 0's result instead of the block it has to factor.
// The first failing pivot (1-based, global) is recorded in *info; later steps see it and
// return immediately.
#include "common.h"

namespace wsic {
namespace {

constexpr int NB = 64;
constexpr int PANEL_WAVES = 8;
constexpr int RPW = NB / PANEL_WAVES;  // rows per wave

// Rows published by the owner of a pivot group: the group's rows of U and of the solved slab X,
// double-buffered by the parity of the group, and the group's first failing pivot (0: none).
struct PanelLds {
  double u[2][RPW][NB];
  double x[2][RPW][NB];
  int bad[2];
};

// v from lane `lane` (uniform) of this wave
__device__ __forceinline__ double lane_bcast(double v, int lane) {
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)bits, lane);
  const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// The pivot loop of one panel workgroup and its stores. a[s], sl[s] hold rows RPW w + s of
// column j of the diagonal block and of this workgroup's slab (block b > 0), as loaded.
// Pivots go in groups of RPW, one group per wave: wave wk holds rows RPW wk .. RPW wk + RPW - 1,
// which have every earlier group's update when its turn comes, so it factors them alone (pivot
// and row entries of its own rows by readlane, no workgroup barrier), solves its slab rows with
// them, and publishes the RPW finished rows of U and X through LDS; after one barrier every wave
// below applies them as one rank-RPW update. Entries left of the diagonal are published as zeros
// and are scratch in the registers.
// The diagonal block (workgroup 0) goes to ud (NB x NB, zeros below the diagonal), not into A:
// other panel workgroups of the same launch may not have read A's copy of it yet.
// pl may alias the memory the caller staged a and sl through: the first barrier orders them.
__device__ __forceinline__ void panel_factor(double (&a)[RPW], double (&sl)[RPW], double* A,
                                             int64_t lda, int64_t kb, int nbk, int64_t n,
                                             int64_t* info, int b, PanelLds* pl, double* ud) {
  const int j = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t c = kb + (int64_t)b * NB + j;  // slab column (b > 0)
  const bool cin = b > 0 && c < n;
  __syncthreads();
#pragma unroll 1
  for (int wk = 0; wk < NB / RPW; ++wk) {
    const int k0 = RPW * wk;
    if (k0 >= nbk) break;  // uniform
    const int par = wk & 1;
    if (w == wk) {
      int bad = 0;
#pragma unroll
      for (int sk = 0; sk < RPW; ++sk) {
        const int k = k0 + sk;
        if (k < nbk) {  // uniform
          const double p = lane_bcast(a[sk], k);
          const bool ok = (p > 0.0) && isfinite(p);
          bad = (bad == 0 && !ok) ? k + 1 : bad;  // a failed pivot ends the factorization below
          // U(k, j) = a(k, j) / sqrt(p) (lane k: sqrt(p)) and X(k, c), with 1/sqrt(p) from the
          // hardware estimate y0 and two Newton steps y1 = y0 f1, y2 = y1 f2, f = 1.5 - (p/2) y^2;
          // the last factor is applied to a y1 and sl y1 so that it is not a step of its own
          const double h = 0.5 * p;
          const double y0 = __builtin_amdgcn_rsq(p);
          const double y1 = y0 * fma(-h * y0, y0, 1.5);
          const double f2 = fma(-h * y1, y1, 1.5);
          const double u = (a[sk] * y1) * f2;
          const double x = (sl[sk] * y1) * f2;
          a[sk] = (j >= k) ? u : 0.0;
          sl[sk] = x;
#pragma unroll
          for (int s = sk + 1; s < RPW; ++s) {
            const double uks = lane_bcast(u, k0 + s);  // U(k, k0 + s)
            a[s] = fma(-uks, u, a[s]);
            sl[s] = fma(-uks, x, sl[s]);
          }
        }
      }
#pragma unroll
      for (int s = 0; s < RPW; ++s) {
        pl->u[par][s][j] = a[s];
        pl->x[par][s][j] = sl[s];
      }
      if (j == 0) pl->bad[par] = bad;
    }
    __syncthreads();
    const int bad = pl->bad[par];
    if (bad != 0) {  // uniform: every thread read the same flag
      if (b == 0 && threadIdx.x == 0) *info = kb + bad;
      return;
    }
    if (w > wk) {
#pragma unroll
      for (int t = 0; t < RPW; ++t) {
        if (k0 + t < nbk) {  // uniform
          const double ut = pl->u[par][t][j];
          const double xt = pl->x[par][t][j];
          // U(k0 + t, RPW w .. RPW w + RPW - 1): the same 64 bytes for every lane, read as
          // 16-byte pairs (one LDS read per pair instead of per entry)
          const double2* row = reinterpret_cast<const double2*>(&pl->u[par][t][RPW * w]);
          double2 q[RPW / 2];
#pragma unroll
          for (int h = 0; h < RPW / 2; ++h) q[h] = row[h];
#pragma unroll
          for (int s = 0; s < RPW; ++s) {
            const double uis = (s & 1) ? q[s >> 1].y : q[s >> 1].x;
            a[s] = fma(-uis, ut, a[s]);
            sl[s] = fma(-uis, xt, sl[s]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < RPW; ++s) {
    const int i = RPW * w + s;
    if (i < nbk) {
      if (b == 0) {
        if (j < nbk) ud[i * NB + j] = (i <= j) ? a[s] : 0.0;
      } else if (cin) {
        A[(kb + i) * lda + c] = sl[s];
      }
    }
  }
}

__global__ __launch_bounds__(64 * PANEL_WAVES) void k_potrf_panel(double* A, int64_t lda, int64_t kb,
                                                                 int nbk, int64_t n, int64_t* info,
                                                                 double* ud) {
  __shared__ PanelLds pl;
  if (*info != 0) return;
  const int j = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int64_t c = kb + (int64_t)b * NB + j;
  const bool cin = b > 0 && c < n;
  double a[RPW], sl[RPW];
#pragma unroll
  for (int s = 0; s < RPW; ++s) {
    const int i = RPW * w + s;
    a[s] = (i <= j && j < nbk) ? A[(kb + i) * lda + kb + j] : (i == j ? 1.0 : 0.0);
    sl[s] = (cin && i < nbk) ? A[(kb + i) * lda + c] : 0.0;
  }
  panel_factor(a, sl, A, lda, kb, nbk, n, info, b, &pl, ud);
}

// The factored diagonal block of step kb from its slot into A (64 x 64 block, ld NB slot)
__device__ __forceinline__ void put_diag(double* A, int64_t lda, int64_t kb, int nbk,
                                         const double* ud) {
  for (int e = threadIdx.x; e < nbk * NB; e += blockDim.x) {
    const int i = e / NB, j = e - i * NB;
    if (j < nbk) A[(kb + i) * lda + kb + j] = ud[e];
  }
}

__global__ void k_put_diag(double* A, int64_t lda, int64_t kb, int nbk, const double* ud) {
  put_diag(A, lda, kb, nbk, ud);
}

// Trailing update A22 -= X^T X after a block row: X = rows r0 .. r0+63 of A at columns
// c0 .. c0+m-1 (the solved block row), A22 = A[c0.., c0..] (m x m), upper 64 x 64 tiles only.
// A tile's C values are loaded into registers first, then the 64 x 64 column strips of X for
// its rows and columns go global -> LDS directly (global_load_lds_dwordx4, lane l of an
// instruction at byte 16 l) in their natural layout, [k][col], which is already the
// conflict-free layout of the v_mfma_f64_16x16x4 operands (16 lanes read 16 consecutive doubles
// of one k row). Diagonal tiles load one strip. 8 waves in 2 x 4, each 32 x 16 = two fragments.
// Requirements (checked by the launcher): A 16-byte aligned, lda even, c0 even.
namespace cupd {
constexpr int T = 64;
typedef __attribute__((address_space(3))) void lds_void;
typedef double d4 __attribute__((ext_vector_type(4)));
}  // namespace cupd

// strip of X: rows r0 .. r0+63 (k) x columns col0 .. col0+63 of A22, as [k][col] in LDS;
// columns past m repeat the last whole chunk (their results are never stored)
__device__ __forceinline__ void load_strip(const double* A, int64_t lda, int64_t r0, int64_t c0,
                                           int64_t m, int64_t col0, double* dst) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t clast = (m - 1) & ~(int64_t)1;
  // 64 rows x 32 chunks of 16 bytes = 32 instructions, 4 per wave
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int ins = 4 * w + h;
    const int p = 64 * ins + lane;
    const int t = p >> 5, ch = p & 31;
    int64_t cc = col0 + 2 * ch;
    cc = cc < clast ? cc : clast;
    __builtin_amdgcn_global_load_lds((const void*)(A + (r0 + t) * lda + c0 + cc),
                                     (cupd::lds_void*)(dst + 128 * ins), 16, 0, 0);
  }
}

// this wave's part of Xa^T Xb for one tile: rows 32 wm + 16 i + lk + 4 r, column 16 wn + lr
__device__ __forceinline__ void tile_mfma(const double (*Xa)[cupd::T], const double (*Xb)[cupd::T],
                                          cupd::d4 (&acc)[2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3, lr = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i] = (cupd::d4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int k4 = 0; k4 < cupd::T / 4; ++k4) {
    const int k = 4 * k4 + lk;
    const double bv = Xb[k][wn * 16 + lr];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(Xa[k][wm * 32 + i * 16 + lr], bv, acc[i], 0, 0, 0);
  }
}

// One step of the right-looking loop in one launch. X is the solved block row [kb, kb+64),
// A22 = A[c0.., c0..] with c0 = kb + 64 and m = n - c0.
//   workgroups 0 .. t-1 (t = ceil(m/64)): the next panel. Workgroup b first applies this step's
//     update to tiles (0, 0) and (0, b) of A22 (the next diagonal block and its slab), passes
//     them through LDS into the pivot layout and factors exactly as k_potrf_panel does;
//   the others: the update of the tiles (tm, tn), 1 <= tm <= tn.
// The next panel needs only the first tile row of this update, so its pivot chain runs beside
// the bulk of the update instead of after it.
__global__ __launch_bounds__(64 * PANEL_WAVES) void k_chol_step(double* A, int64_t lda, int64_t kb,
                                                               int64_t n, int npanel,
                                                               int64_t* info, const double* ud_cur,
                                                               double* ud_next) {
  using namespace cupd;
  static_assert(PANEL_WAVES == 8, "tile layout: 8 waves in 2 x 4");
  __shared__ __attribute__((aligned(1024))) double Xs[2][T][T];
  static_assert(sizeof(PanelLds) <= sizeof(Xs), "panel rows live in the operand strips");
  if (*info != 0) return;
  const int64_t c0 = kb + NB, m = n - c0;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3, lr = lane & 15, lk = lane >> 4;
  const int bid = blockIdx.x;

  if (bid < npanel) {
    const int b = bid;
    const int64_t j0 = (int64_t)b * T;
    // this step's factored diagonal block into A (nothing in this launch reads that block)
    if (b == 0) put_diag(A, lda, kb, NB, ud_cur);
    double cd[2][4], cs[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t ii = wm * 32 + i * 16 + lk + 4 * r, jj = wn * 16 + lr;
        cd[i][r] = (ii < m && jj < m) ? A[(c0 + ii) * lda + c0 + jj] : 0.0;
        cs[i][r] = (b > 0 && ii < m && j0 + jj < m) ? A[(c0 + ii) * lda + c0 + j0 + jj] : 0.0;
      }
    load_strip(A, lda, kb, c0, m, 0, &Xs[0][0][0]);
    if (b > 0) load_strip(A, lda, kb, c0, m, j0, &Xs[1][0][0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    d4 ad[2], as[2];
    tile_mfma(Xs[0], Xs[0], ad);
    if (b > 0) tile_mfma(Xs[0], Xs[1], as);
    __syncthreads();  // every wave done with the strips
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = wm * 32 + i * 16 + lk + 4 * r, jj = wn * 16 + lr;
        Xs[0][ii][jj] = cd[i][r] - ad[i][r];
        if (b > 0) Xs[1][ii][jj] = cs[i][r] - as[i][r];
      }
    __syncthreads();
    const int nbk = (int)(m < NB ? m : NB);
    const int j = lane;
    const bool cin = b > 0 && c0 + j0 + j < n;
    double a[RPW], sl[RPW];
#pragma unroll
    for (int s = 0; s < RPW; ++s) {
      const int i = RPW * w + s;
      a[s] = (i <= j && j < nbk) ? Xs[0][i][j] : (i == j ? 1.0 : 0.0);
      sl[s] = (cin && i < nbk) ? Xs[1][i][j] : 0.0;
    }
    panel_factor(a, sl, A, lda, c0, nbk, n, info, b, reinterpret_cast<PanelLds*>(&Xs[0][0][0]),
                 ud_next);
    return;
  }

  // update tile (tm, tn), 1 <= tm <= tn: triangular index over the tiles below the first row
  const int64_t u = bid - npanel;
  int64_t tn = (int64_t)((sqrt(8.0 * (double)u + 1.0) - 1.0) * 0.5);
  while ((tn + 1) * (tn + 2) / 2 <= u) ++tn;
  while (tn * (tn + 1) / 2 > u) --tn;
  const int64_t tm = u - tn * (tn + 1) / 2 + 1;
  ++tn;
  const int64_t i0 = tm * T, j0 = tn * T;
  const bool diag = (tm == tn);
  double cold[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t ii = i0 + wm * 32 + i * 16 + lk + 4 * r, jj = j0 + wn * 16 + lr;
      cold[i][r] = (ii < m && jj < m) ? A[(c0 + ii) * lda + c0 + jj] : 0.0;
    }
  load_strip(A, lda, kb, c0, m, i0, &Xs[0][0][0]);
  if (!diag) load_strip(A, lda, kb, c0, m, j0, &Xs[1][0][0]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  d4 acc[2];
  tile_mfma(Xs[0], diag ? Xs[0] : Xs[1], acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t ii = i0 + wm * 32 + i * 16 + lk + 4 * r, jj = j0 + wn * 16 + lr;
      if (ii < m && jj < m) A[(c0 + ii) * lda + c0 + jj] = cold[i][r] - acc[i][r];
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
                       double* ud, hipStream_t st) {
  if (nbk <= 0 || nbk > NB) {
    set_error("internal: potrf block %d", nbk);
    return WSIC_E_INVAL;
  }
  const int64_t m = n - kb - nbk;  // columns right of the diagonal block
  const unsigned blocks = 1 + (unsigned)((m + NB - 1) / NB);
  const double work = (double)nbk * nbk * nbk / 3.0 + (double)nbk * nbk * m;
  WSIC_LAUNCH("potrf_panel", work, st, k_potrf_panel, dim3(blocks), dim3(64 * PANEL_WAVES), 0, A, lda, kb, nbk, n,
              info, ud);
  return WSIC_OK;
}

int launch_put_diag(double* A, int64_t lda, int64_t kb, int nbk, const double* ud, hipStream_t st) {
  WSIC_LAUNCH("put_diag", 16.0 * nbk * nbk, st, k_put_diag, dim3(1), dim3(256), 0, A, lda, kb, nbk, ud);
  return WSIC_OK;
}

bool chol_step_ok(const double* A, int64_t lda, int64_t c0) {
  return (((uintptr_t)A) & 15) == 0 && (lda % 2) == 0 && (c0 % 2) == 0;
}

int launch_chol_step(double* A, int64_t lda, int64_t kb, int64_t n, int64_t* info,
                     const double* ud_cur, double* ud_next, hipStream_t st) {
  const int64_t c0 = kb + NB, m = n - c0;
  if (m <= 0 || !chol_step_ok(A, lda, c0)) {
    set_error("internal: cholesky step preconditions");
    return WSIC_E_INVAL;
  }
  const int64_t t = (m + NB - 1) / NB;  // panel workgroups: the first tile row of the update
  const int64_t tiles = t * (t + 1) / 2;
  const double nbk = (double)(m < NB ? m : NB);
  const double work = (double)m * (double)(m + 1) * NB + nbk * nbk * nbk / 3.0 + nbk * nbk * (m - nbk);
  WSIC_LAUNCH("chol_step", work, st, k_chol_step, dim3((unsigned)tiles), dim3(64 * PANEL_WAVES), 0,
              A, lda, kb, n, (int)t, info, ud_cur, ud_next);
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
