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
      if (k < K && n < g.N) bv = KMAJOR ? g.B[k * g.ldb + n] : g.B[n * g.ldb + k];
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
