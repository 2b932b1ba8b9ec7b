// Exact integer form of the SIC interference product on int8 matrix cores.
//
// The interference of finished columns R on pending columns L is
//     G[r, j] += sum_{k in R} B_jk q_rk ,  B_jk = U_jk / U_kk ,
// a product of the integer codes with a matrix that does not depend on the grid scale c
// (the Babai form of the WaterSIC page's SIC, Sommario tecnico §2 item 1). Here each row j of B
// is written in fixed point with a power-of-two scale, B_jk ~ 2^(e_j - P) Bt_jk, where
// |B_jk| < 2^e_j, Bt_jk = rint(B_jk 2^(P - e_j)) and P = 8 NL - 2, and Bt is split into NL
// balanced base-256 digits (int8 planes D_0 .. D_{NL-1}, most significant first). Codes enter
// as int8 (clamped to +-127; the excess of the rare larger codes is handled exactly in the
// SIC leaf). v_mfma_i32_32x32x32_i8 then accumulates every digit product exactly in int32, and
// only the final combination F = 2^(e_j-P) sum_l 256^(NL-1-l) acc_l is rounded (fp64).
// The one approximation is Bt's rounding: |error| <= 2^(e_j - P - 1) sum_k |q_rk|, a bound the
// leaf uses to re-derive in fp64 the rare rounding decisions that fall inside it.
//
// MFMA i32 32x32x32 i8 lane layout (checked on gfx950): A operand lane l holds the 16 bytes
// A[l%32][16*(l/32) + e], B operand B[16*(l/32) + e][l%32], result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "common.h"

namespace wsic {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int NL = LIMBS;
constexpr int P = 8 * NL - 2;

// e_j: smallest power of two strictly above max_{k>j} |B_jk| (0 when the row is empty).
// One workgroup per row.
__global__ __launch_bounds__(256) void k_row_scale(const double* __restrict__ U, int64_t ldu,
                                                   int64_t n, const double* __restrict__ invd,
                                                   double* __restrict__ escale,
                                                   double* __restrict__ bscale) {
  __shared__ double red[256];
  const int64_t j = blockIdx.x;
  double m = 0.0;
  for (int64_t k = j + 1 + threadIdx.x; k < n; k += 256) m = fmax(m, fabs(U[j * ldu + k] * invd[k]));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mx = red[0];
    const int e = (mx > 0.0) ? ilogb(mx) + 1 : 0;
    escale[j] = ldexp(1.0, e - P);
    bscale[j] = ldexp(1.0, e);
  }
}

// Digit planes: D[l][j][k] for k > j, zero elsewhere (including the padding k in [n, ldd)).
__global__ void k_limb_digits(const double* __restrict__ U, int64_t ldu, int64_t n,
                              const double* __restrict__ invd, const double* __restrict__ escale,
                              int8_t* __restrict__ D, int64_t ldd) {
  const int64_t j = blockIdx.y;
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= ldd) return;
  long long x = 0;
  if (k > j && k < n) {
    // B_jk * 2^(P - e_j): exact power-of-two scaling, then one rounding
    const double v = (U[j * ldu + k] * invd[k]) / escale[j];
    x = (long long)rint(v);
  }
  const int64_t plane = n * ldd;
#pragma unroll
  for (int l = NL - 1; l >= 0; --l) {
    long long d = x & 255;  // balanced digit in [-128, 127]
    if (d >= 128) d -= 256;
    x = (x - d) / 256;
    D[(int64_t)l * plane + j * ldd + k] = (int8_t)d;
  }
}

// C[M x N] (+)= F, F(m, n) = escale[n] * sum_l 256^(NL-1-l) sum_k A8(m,k) D_l(n,k).
// Tile 128 x 64, K-step 64; 4 waves in 2 x 2, each 64 x 32 = two 32x32 fragments, every
// fragment with NL int32 accumulators. A8 rows and D rows are 16-byte aligned with zero
// padding past the layer, so every load is a whole 16-byte vector.
constexpr int TM = 128, TN = 64, TKB = 64;
constexpr int LROW = TKB + 16;  // LDS row length in bytes (keeps 16-byte alignment)

__global__ __launch_bounds__(256) void k_gemm_i8(int64_t M, int64_t N, int64_t K,
                                                 const int8_t* __restrict__ A8, int64_t lda,
                                                 const int8_t* __restrict__ D, int64_t ldd,
                                                 int64_t plane, const double* __restrict__ escale,
                                                 double* __restrict__ C, int64_t ldc, double beta,
                                                 int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t As[TM][LROW];
  __shared__ __attribute__((aligned(16))) int8_t Bs[NL][TN][LROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * TM, n0 = tn * TN;
  const int wm = wave >> 1, wn = wave & 1;

  // loaders: A 128 rows x 64 bytes = two 16-byte vectors per thread; each D plane 64 rows x
  // 64 bytes = one vector per thread
  const int ar = tid >> 1, ac = (tid & 1) * 32;
  const int br = tid >> 2, bc = (tid & 3) * 16;
  uint4 pa[2], pb[NL];
  auto fetch = [&](int64_t k0) {
    const int64_t m = m0 + ar;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      pa[h] = (m < M && k0 + ac + 16 * h < K)
                  ? *reinterpret_cast<const uint4*>(A8 + m * lda + k0 + ac + 16 * h)
                  : make_uint4(0, 0, 0, 0);
    const int64_t nn = n0 + br;
#pragma unroll
    for (int l = 0; l < NL; ++l)
      pb[l] = (nn < N && k0 + bc < K)
                  ? *reinterpret_cast<const uint4*>(D + l * plane + nn * ldd + k0 + bc)
                  : make_uint4(0, 0, 0, 0);
  };
  auto stash = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h) *reinterpret_cast<uint4*>(&As[ar][ac + 16 * h]) = pa[h];
#pragma unroll
    for (int l = 0; l < NL; ++l) *reinterpret_cast<uint4*>(&Bs[l][br][bc]) = pb[l];
  };

  v16i acc[2][NL];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int l = 0; l < NL; ++l) acc[i][l] = (v16i){};

  fetch(0);
  for (int64_t k0 = 0; k0 < K; k0 += TKB) {
    __syncthreads();
    stash();
    __syncthreads();
    if (k0 + TKB < K) fetch(k0 + TKB);
#pragma unroll
    for (int ks = 0; ks < TKB / 32; ++ks) {
      const int kb = ks * 32 + 16 * (lane >> 5);
      v4i a[2], b[NL];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const v4i*>(&As[wm * 64 + i * 32 + (lane & 31)][kb]);
#pragma unroll
      for (int l = 0; l < NL; ++l)
        b[l] = *reinterpret_cast<const v4i*>(&Bs[l][wn * 32 + (lane & 31)][kb]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int l = 0; l < NL; ++l)
          acc[i][l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[l], acc[i][l], 0, 0, 0);
    }
  }

  const int64_t n = n0 + wn * 32 + (lane & 31);
  if (n >= N) return;
  const double es = escale[n];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m < M) {
        double f = 0.0;
#pragma unroll
        for (int l = 0; l < NL; ++l) f = fma((double)acc[i][l][r], ldexp(1.0, 8 * (NL - 1 - l)), f);
        f *= es;
        double* p = C + m * ldc + n;
        *p = (beta != 0.0) ? fma(beta, *p, f) : f;
      }
    }
}

}  // namespace

int launch_limb_pack(const double* U, int64_t ldu, int64_t n, const double* invd, double* escale,
                     double* bscale, int8_t* D, int64_t ldd, hipStream_t st) {
  WSIC_LAUNCH("limb_scale", 8.0 * n * n / 2, st, k_row_scale, dim3((unsigned)n), dim3(256), 0, U,
              ldu, n, invd, escale, bscale);
  WSIC_LAUNCH("limb_digits", (double)n * ldd * (4.0 + NL), st, k_limb_digits,
              dim3((unsigned)((ldd + 255) / 256), (unsigned)n), dim3(256), 0, U, ldu, n, invd,
              escale, D, ldd);
  return WSIC_OK;
}

int launch_gemm_i8(int64_t M, int64_t N, int64_t K, const int8_t* A8, int64_t lda, const int8_t* D,
                   int64_t ldd, int64_t plane, const double* escale, double* C, int64_t ldc,
                   double beta, hipStream_t st) {
  if (M <= 0 || N <= 0) return WSIC_OK;
  if ((lda % 16) || (ldd % 16) || (((uintptr_t)A8) & 15) || (((uintptr_t)D) & 15)) {
    set_error("internal: int8 operands must be 16-byte aligned");
    return WSIC_E_INVAL;
  }
  const int64_t tiles_n = (N + TN - 1) / TN, tiles = ((M + TM - 1) / TM) * tiles_n;
  // algorithmic int8 ops: NL digit products per multiply-add
  const double work = 2.0 * NL * (double)M * (double)N * (double)K;
  WSIC_LAUNCH("gemm_trail_i8", work, st, k_gemm_i8, dim3((unsigned)tiles), dim3(256), 0, M, N, K,
              A8, lda, D, ldd, plane, escale, C, ldc, beta, (int)tiles_n);
  return WSIC_OK;
}

}  // namespace wsic
