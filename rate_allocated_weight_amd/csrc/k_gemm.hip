// fp64 MFMA GEMM family on gfx950 (v_mfma_f64_16x16x4_f64).
//
//   C[M x N] = beta * C + alpha * sum_k A'(m, k) * B(n, k)
//
// Uses in the library:
//   * Y = W U^T                    (A = W in f32/bf16, B = U upper: tri)
//   * G[:, L] (+)= (Q diag(1/U_kk))[:, R] U[L, R]^T   (SIC interference of a finished column
//                                                     range R on the pending range L)
//   * A22 -= P^T P                 (Cholesky trailing update, operands stored k-major)
//   * ||(W - W_hat) U^T||_F^2      (direct distortion, sum-of-squares epilogue)
//
// Tile TM x TN x 16 per 256-thread workgroup (128 x 128 when the product has enough tiles to
// fill the chip twice over, else 64 x 64); 4 waves in a 2 x 2 grid, each a (TM/2) x (TN/2)
// block of 16 x 16 MFMA accumulators. Operands are staged in LDS k-major ([k][m], [k][n]) so
// that the 64 lanes of an MFMA read 4 k-rows x 16 consecutive doubles. Global tiles are
// prefetched into registers one k-step ahead (register double buffering).
//
// MFMA f64 16x16x4 lane layout (checked on gfx950): A operand lane l = A[l%16][l/16],
// B operand lane l = B[l/16][l%16], result register r of lane l = D[l/16 + 4r][l%16].
#include "common.h"
#include "pipe.h"

namespace wsic {
namespace {

constexpr int TK = 16;
constexpr int LDS_PAD = 2;  // doubles of padding per k-row
typedef double d4 __attribute__((ext_vector_type(4)));

template <int AMODE>
__device__ __forceinline__ double load_a(const GemmArgs& g, int64_t m, int64_t k) {
  if (AMODE == A_F64) return ((const double*)g.A)[m * g.lda + k];
  if (AMODE == A_F32) return (double)((const float*)g.A)[m * g.lda + k];
  if (AMODE == A_BF16) return (double)bf16_to_f32(((const uint16_t*)g.A)[m * g.lda + k]);
  if (AMODE == A_CODES) return g.vec[k] * (double)((const int32_t*)g.A)[m * g.lda + k];
  if (AMODE == A_ERR_F32)
    return (double)((const float*)g.A)[m * g.lda + k] - g.vec[k] * (double)g.Q[m * g.ldq + k];
  if (AMODE == A_ERR_BF16)
    return (double)bf16_to_f32(((const uint16_t*)g.A)[m * g.lda + k]) -
           g.vec[k] * (double)g.Q[m * g.ldq + k];
  if (AMODE == A_F64_T) return ((const double*)g.A)[k * g.lda + m];
  return 0.0;
}

template <int AMODE, int EPI, int TM, int TN>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g, int tiles_n) {
  constexpr int EA = TM * TK / 256, EB = TN * TK / 256;  // elements per thread per k-step
  constexpr int FM = TM / 32, FN = TN / 32;              // 16x16 fragments per wave
  __shared__ double As[TK][TM + LDS_PAD];
  __shared__ double Bs[TK][TN + LDS_PAD];
  __shared__ double red[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
  const int64_t m0 = tm * TM, n0 = tn * TN;
  if (g.upper_only && n0 + TN - 1 < m0) {
    if (EPI == EPI_SUMSQ && tid == 0) g.partial[tile] = 0.0;
    return;
  }

  int64_t kbeg = 0;
  if (g.tri) kbeg = (n0 / TK) * TK;
  const int64_t K = g.K;

  // loader mapping: k-contiguous operands -> a thread loads EA consecutive k of one row;
  // k-major operands (A_F64_T) -> a thread loads EA consecutive m (n) of one k row.
  constexpr bool KMAJOR = (AMODE == A_F64_T);
  const int ar = KMAJOR ? tid / (TM / EA) : tid / (TK / EA);
  const int ac = KMAJOR ? (tid % (TM / EA)) * EA : (tid % (TK / EA)) * EA;
  const int br = KMAJOR ? tid / (TN / EB) : tid / (TK / EB);
  const int bc = KMAJOR ? (tid % (TN / EB)) * EB : (tid % (TK / EB)) * EB;

  double pa[EA], pb[EB];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int e = 0; e < EA; ++e) {
      const int64_t m = KMAJOR ? m0 + ac + e : m0 + ar;
      const int64_t k = KMAJOR ? k0 + ar : k0 + ac + e;
      pa[e] = (k < K && m < g.M) ? load_a<AMODE>(g, m, k) : 0.0;
    }
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      const int64_t n = KMAJOR ? n0 + bc + e : n0 + br;
      const int64_t k = KMAJOR ? k0 + br : k0 + bc + e;
      double bv = 0.0;
      // with tri, B(n, k) below the diagonal (k < n) is zero whatever memory holds there
      if (k < K && n < g.N && !(g.tri && k < n)) bv = KMAJOR ? g.B[k * g.ldb + n] : g.B[n * g.ldb + k];
      pb[e] = bv;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int e = 0; e < EA; ++e) {
      if (KMAJOR)
        As[ar][ac + e] = pa[e];
      else
        As[ac + e][ar] = pa[e];
    }
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      if (KMAJOR)
        Bs[br][bc + e] = pb[e];
      else
        Bs[bc + e][br] = pb[e];
    }
  };

  d4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (d4){0.0, 0.0, 0.0, 0.0};

  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 15, lk = lane >> 4;

  if (kbeg < K) fetch(kbeg);
  for (int64_t k0 = kbeg; k0 < K; k0 += TK) {
    __syncthreads();  // previous compute done with LDS
    stash();
    __syncthreads();
    if (k0 + TK < K) fetch(k0 + TK);  // overlaps with the MFMAs below
#pragma unroll
    for (int kk = 0; kk < TK / 4; ++kk) {
      const int kr = kk * 4 + lk;
      double a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = As[kr][wm * (TM / 2) + i * 16 + lrow];
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = Bs[kr][wn * (TN / 2) + j * 16 + lrow];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: result register r of lane l sits at row l/16 + 4r, column l%16
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * (TM / 2) + i * 16 + (lane >> 4) + 4 * r;
        const int64_t n = n0 + wn * (TN / 2) + j * 16 + (lane & 15);
        if (m < g.M && n < g.N) {
          const double v = acc[i][j][r];
          if (EPI == EPI_STORE) {
            double* p = g.C + m * g.ldc + n;
            *p = (g.beta != 0.0) ? fma(g.alpha, v, g.beta * *p) : g.alpha * v;
          } else {
            ss = fma(v, v, ss);
          }
        }
      }
  if (EPI == EPI_SUMSQ) {
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_down(ss, off, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    if (tid == 0) g.partial[tile] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

// Y = A B^T for the SIC setup, A = W (bf16 or fp32, row-major M x K), B = U (fp64 row-major,
// B(n, k) = U[n][k], zero for k < n: each N-tile starts its K loop at its first column and masks
// the strict lower triangle at operand read, so U's lower triangle is never used).
//
// Tile 128 x 128 x 16 per 256-thread workgroup; 4 waves in 2 x 2, each 64 x 64 = 4 x 4 fragments
// of v_mfma_f64_16x16x4. Operands go global -> LDS directly (global_load_lds_dwordx4, lane l of a
// wave's instruction at byte 16 l) through a ring of 3 buffers, so two K-steps are in flight while
// one is multiplied; A stays in its storage type in LDS and is widened to fp64 at operand read.
// LDS layouts (16-byte chunks): A chunk c of row m at slot c * 128 + m (so the 16 rows of one
// operand read fall in distinct banks); B chunk c of row n at slot 8 n + (c ^ (n & 7)).
// Tiles are ordered N-major: the long tiles (small n0, K from n0) are dispatched first.
// Requirements (checked by the launcher): K % 16 == 0, A and B 16-byte aligned with row pitches
// that keep every chunk aligned.
namespace ydma {
constexpr int TM = 128, TN = 128, TKY = 16, STAGES = 3;
constexpr int B_BYTES = TN * TKY * 8;  // 16 KiB
template <typename TA>
__device__ __forceinline__ double widen(TA v);
template <>
__device__ __forceinline__ double widen<uint16_t>(uint16_t v) {
  return (double)bf16_to_f32(v);
}
template <>
__device__ __forceinline__ double widen<float>(float v) {
  return (double)v;
}
}  // namespace ydma

template <typename TA>
__global__ __launch_bounds__(256) void k_gemm_y(int64_t M, int64_t N, int64_t K,
                                                const TA* __restrict__ A, int64_t lda,
                                                const double* __restrict__ B, int64_t ldb,
                                                double* __restrict__ C, int64_t ldc, int tiles_m) {
  using namespace ydma;
  constexpr int EC = 16 / (int)sizeof(TA);     // A elements per chunk
  constexpr int A_CH = TKY / EC;                // A chunks per row per K-step
  constexpr int A_BYTES = TM * TKY * (int)sizeof(TA);
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_INS = A_BYTES / 4096, B_INS = B_BYTES / 4096;  // per wave per stage
  constexpr int DMA = A_INS + B_INS;
  static_assert(A_INS * 4096 == A_BYTES && B_INS * 4096 == B_BYTES, "whole DMA rounds");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tn = blockIdx.x / tiles_m, tm = blockIdx.x % tiles_m;
  const int64_t m0 = tm * TM, n0 = tn * TN;
  const int wm = wave >> 1, wn = wave & 1;

  const TA* asrc[A_INS];
  const double* bsrc[B_INS];
  int aoff[A_INS], boff[B_INS];
#pragma unroll
  for (int h = 0; h < A_INS; ++h) {
    const int p = 64 * (A_INS * wave + h) + lane;  // chunk slot
    const int c = p / TM, m = p % TM;
    const int64_t mg = (m0 + m < M) ? m0 + m : M - 1;
    asrc[h] = A + mg * lda + EC * c;
    aoff[h] = 1024 * (A_INS * wave + h);
  }
#pragma unroll
  for (int h = 0; h < B_INS; ++h) {
    const int p = 64 * (B_INS * wave + h) + lane;
    const int n = p >> 3, c = (p & 7) ^ (n & 7);
    const int64_t ng = (n0 + n < N) ? n0 + n : N - 1;
    bsrc[h] = B + ng * ldb + 2 * c;
    boff[h] = A_BYTES + 1024 * (B_INS * wave + h);
  }
  auto issue = [&](int64_t k0, int buf) {
    char* base = smem + buf * STAGE;
#pragma unroll
    for (int h = 0; h < A_INS; ++h)
      pipe::dma16(asrc[h] + k0, base + aoff[h]);
#pragma unroll
    for (int h = 0; h < B_INS; ++h)
      pipe::dma16(bsrc[h] + k0, base + boff[h]);
  };

  d4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (d4){0.0, 0.0, 0.0, 0.0};

  const int lr = lane & 15, lk = lane >> 4;
  const int64_t kbeg = n0;  // B(n, k) = 0 for k < n0 in this tile
  const int nk = (int)((K - kbeg) / TKY);
  if (nk > 0) issue(kbeg, 0);
  if (nk > 1) issue(kbeg + TKY, 1);
  int cur = 0, nxt = 2;
  for (int t = 0; t < nk; ++t) {
    pipe::wait_ahead<DMA, STAGES - 2>(min(STAGES - 2, nk - 1 - t));
    pipe::barrier_lds();
    if (t + 2 < nk) issue(kbeg + (int64_t)(t + 2) * TKY, nxt);
    const char* As = smem + cur * STAGE;
    const char* Bs = As + A_BYTES;
    cur = (cur == STAGES - 1) ? 0 : cur + 1;
    nxt = (nxt == STAGES - 1) ? 0 : nxt + 1;
    const int64_t k0 = kbeg + (int64_t)t * TKY;
#pragma unroll
    for (int kk = 0; kk < TKY / 4; ++kk) {
      const int k = kk * 4 + lk;  // this lane's k within the step
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 64 + i * 16 + lr;
        const TA* pa = reinterpret_cast<const TA*>(As + ((k / EC) * TM + m) * 16) + (k % EC);
        a[i] = widen<TA>(*pa);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 64 + j * 16 + lr;
        const double* pb =
            reinterpret_cast<const double*>(Bs + (8 * n + ((k >> 1) ^ (n & 7))) * 16) + (k & 1);
        b[j] = (k0 + k >= n0 + n) ? *pb : 0.0;  // strict lower triangle of U reads as zero
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  (void)A_CH;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + i * 16 + lk + 4 * r;
        const int64_t n = n0 + wn * 64 + j * 16 + lr;
        if (m < M && n < N) C[m * ldc + n] = acc[i][j][r];
      }
}

// The 128 x 128 tile runs one wave per SIMD (200 VGPRs + 128 AGPRs) and measured slower than
// 64 x 64 on gfx950 for every product size here; it stays compiled but unused.
bool use_big(const GemmArgs& g) {
  (void)g;
  return false;
}

template <int AMODE, int EPI>
int launch_one(const GemmArgs& g, const char* family, double work, hipStream_t st) {
  if (use_big(g)) {
    const int64_t tiles_n = (g.N + 127) / 128, tiles = ((g.M + 127) / 128) * tiles_n;
    WSIC_LAUNCH(family, work, st, (k_gemm<AMODE, EPI, 128, 128>), dim3((unsigned)tiles),
                dim3(256), 0, g, (int)tiles_n);
  } else {
    const int64_t tiles_n = (g.N + 63) / 64, tiles = ((g.M + 63) / 64) * tiles_n;
    WSIC_LAUNCH(family, work, st, (k_gemm<AMODE, EPI, 64, 64>), dim3((unsigned)tiles), dim3(256),
                0, g, (int)tiles_n);
  }
  return WSIC_OK;
}

}  // namespace

int launch_gemm_y(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                  const double* B, int64_t ldb, double* C, int64_t ldc, double work, hipStream_t st) {
  if (M <= 0 || N <= 0) return WSIC_OK;
  const int64_t esz = (dtype == WSIC_BF16) ? 2 : 4;
  const bool dma_ok = K % ydma::TKY == 0 && (((uintptr_t)A) & 15) == 0 && ((lda * esz) % 16) == 0 &&
                      (((uintptr_t)B) & 15) == 0 && ((ldb * 8) % 16) == 0;
  if (!dma_ok) {
    GemmArgs g{};
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = A;
    g.lda = lda;
    g.B = B;
    g.ldb = ldb;
    g.C = C;
    g.ldc = ldc;
    g.alpha = 1.0;
    g.beta = 0.0;
    g.tri = 1;
    return launch_gemm(dtype == WSIC_BF16 ? A_BF16 : A_F32, EPI_STORE, g, "gemm_y", work, st);
  }
  const int64_t tiles_m = (M + ydma::TM - 1) / ydma::TM, tiles = tiles_m * ((N + ydma::TN - 1) / ydma::TN);
  if (dtype == WSIC_BF16)
    WSIC_LAUNCH("gemm_y", work, st, k_gemm_y<uint16_t>, dim3((unsigned)tiles), dim3(256), 0, M, N, K,
                (const uint16_t*)A, lda, B, ldb, C, ldc, (int)tiles_m);
  else
    WSIC_LAUNCH("gemm_y", work, st, k_gemm_y<float>, dim3((unsigned)tiles), dim3(256), 0, M, N, K,
                (const float*)A, lda, B, ldb, C, ldc, (int)tiles_m);
  return WSIC_OK;
}

int gemm_tiles(const GemmArgs& g) {
  if (use_big(g)) return (int)(((g.M + 127) / 128) * ((g.N + 127) / 128));
  return (int)(((g.M + 63) / 64) * ((g.N + 63) / 64));
}

int launch_gemm(int amode, int epi, const GemmArgs& g, const char* family, double work,
                hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return WSIC_OK;
#define WSIC_GEMM_CASE(AM)                                                  \
  case AM:                                                                  \
    return epi == EPI_STORE ? launch_one<AM, EPI_STORE>(g, family, work, st) \
                            : launch_one<AM, EPI_SUMSQ>(g, family, work, st);
  switch (amode) {
    WSIC_GEMM_CASE(A_F64)
    WSIC_GEMM_CASE(A_F32)
    WSIC_GEMM_CASE(A_BF16)
    WSIC_GEMM_CASE(A_CODES)
    WSIC_GEMM_CASE(A_ERR_F32)
    WSIC_GEMM_CASE(A_ERR_BF16)
    WSIC_GEMM_CASE(A_F64_T)
    default:
      set_error("internal: bad gemm mode %d", amode);
      return WSIC_E_INVAL;
  }
#undef WSIC_GEMM_CASE
}

}  // namespace wsic
