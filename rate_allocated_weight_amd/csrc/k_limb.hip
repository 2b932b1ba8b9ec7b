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
#include "pipe.h"

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
// Four adjacent k per thread (ldd is a multiple of 128), one 4-byte store per plane; x - d is a
// multiple of 256, so the shift is the exact division.
__global__ void k_limb_digits(const double* __restrict__ U, int64_t ldu, int64_t n,
                              const double* __restrict__ invd, const double* __restrict__ escale,
                              int8_t* __restrict__ D, int64_t ldd) {
  const int64_t j = blockIdx.y;
  const int64_t k0 = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (k0 >= ldd) return;
  const double ies = 1.0 / escale[j];  // exact: escale is a power of two
  uint32_t w[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) w[l] = 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t k = k0 + c;
    long long x = 0;
    if (k > j && k < n) {
      // B_jk * 2^(P - e_j): exact power-of-two scaling, then one rounding
      const double v = (U[j * ldu + k] * invd[k]) * ies;
      x = (long long)rint(v);
    }
#pragma unroll
    for (int l = NL - 1; l >= 0; --l) {
      long long d = x & 255;  // balanced digit in [-128, 127]
      if (d >= 128) d -= 256;
      x = (x - d) >> 8;
      w[l] |= ((uint32_t)(d & 255)) << (8 * c);
    }
  }
  const int64_t plane = n * ldd;
#pragma unroll
  for (int l = 0; l < NL; ++l)
    *reinterpret_cast<uint32_t*>(D + (int64_t)l * plane + j * ldd + k0) = w[l];
}

// C[M x N] (+)= F, F(m, n) = escale[n] * sum_l 256^(NL-1-l) sum_k A8(m,k) D_l(n,k).
//
// Tile TM x 64, K-step 64; NW waves in (TM/64) x 2, each 64 x 32 = two 32x32 fragments, every
// fragment with NL int32 accumulators. Two shapes: 128 x 64 with 4 waves, and 256 x 64 with 8
// waves (two per SIMD) for the large products, where it reads 36 KiB of operands per K-step for
// twice the multiply-adds of the 28 KiB small tile (the product is bound by the operand traffic
// from L2: each digit plane is read once per 64-row strip of codes). Operands go from global
// memory straight into LDS (global_load_lds_dwordx4: each instruction of a wave fills 1 KiB, lane
// l at byte 16 l) through a ring of STAGES buffers, so STAGES - 1 K-steps are in flight while one
// is multiplied, and no registers are spent on staging. A stage's 1 KiB loads are dealt to the
// waves round-robin (so with 36 of them, waves 0-3 issue 5 and waves 4-7 issue 4, and each waits
// on its own count). Each 64-byte LDS row holds four 16-byte chunks; chunk c of row r sits in slot
// c ^ swz(r), which spreads the 32 rows one MFMA operand read touches over all LDS banks. When
// beta != 0 the C tile is loaded into registers before the first operand load, so its latency
// hides behind the whole K loop.
//
// Reads are whole 64-byte K-steps: A8 and D must hold zeros in columns [K, roundup(K, 64)).
// Rows past M or N load a clamped (valid) row whose results are never stored.
constexpr int TN = 64, TKB = 64;
constexpr int STAGES = 3;

template <int TM_, int NW_>
struct I8Tile {
  static constexpr int TM = TM_, NW = NW_;
  static constexpr int A_BYTES = TM * TKB;
  static constexpr int B_BYTES = NL * TN * TKB;  // 20 KiB
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_INS = A_BYTES / 1024, INS = STAGE_BYTES / 1024;  // 1 KiB loads per stage
  static constexpr int DMA_MAX = (INS + NW - 1) / NW;                     // per wave (at most)
  // the C tile goes into registers before the K loop when the registers allow (the large tile's
  // 160 accumulator registers per lane leave no room: it loads C after the loop)
  static constexpr bool C_FIRST = NW == 4;
  static_assert(TM == 64 * (NW / 2) && NW % 2 == 0, "waves in (TM/64) x 2");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 4096 == 0, "whole 1 KiB loads");
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <class Cfg>
__global__ __launch_bounds__(64 * Cfg::NW) void k_gemm_i8(int64_t M, int64_t N, int64_t K,
                                                          const int8_t* __restrict__ A8,
                                                          int64_t lda,
                                                          const int8_t* __restrict__ D,
                                                          int64_t ldd, int64_t plane,
                                                          const double* __restrict__ escale,
                                                          double* __restrict__ C, int64_t ldc,
                                                          double beta, int tiles_n) {
  constexpr int TM = Cfg::TM, NW = Cfg::NW, A_BYTES = Cfg::A_BYTES, A_INS = Cfg::A_INS;
  constexpr int INS = Cfg::INS, DMA_MAX = Cfg::DMA_MAX, STAGE_BYTES = Cfg::STAGE_BYTES;
  __shared__ __attribute__((aligned(1024))) int8_t smem[STAGES * STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * TM, n0 = tn * TN;
  const int wm = wave >> 1, wn = wave & 1;

  // C tile of this lane (result layout of the 32x32 fragments), loaded first when accumulating
  const int64_t ncol = n0 + wn * 32 + (lane & 31);
  const bool ncol_ok = ncol < N;
  double cold[2][16];
  auto load_c = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        cold[i][r] = (m < M && ncol_ok) ? C[m * ldc + ncol] : 0.0;
      }
  };
  if (Cfg::C_FIRST && beta != 0.0) load_c();

  // DMA sources of this lane: load g = wave + NW h of a stage; g < A_INS covers rows 16 g + l/4
  // of the codes, the rest limb plane (g - A_INS) / 4, rows 16 ((g - A_INS) % 4) + l/4 of D
  const int8_t* src[DMA_MAX];
  int off[DMA_MAX];
#pragma unroll
  for (int h = 0; h < DMA_MAX; ++h) {
    int g = wave + NW * h;
    g = g < INS ? g : INS - 1;  // (not issued: see `mine` below)
    if (g < A_INS) {
      const int r = 16 * g + (lane >> 2);
      const int c = (lane & 3) ^ swz(r);
      const int64_t m = (m0 + r < M) ? m0 + r : M - 1;
      src[h] = A8 + m * lda + 16 * c;
    } else {
      const int bi = g - A_INS;
      const int l = bi >> 2, r = 16 * (bi & 3) + (lane >> 2);
      const int c = (lane & 3) ^ swz(r);
      const int64_t n = (n0 + r < N) ? n0 + r : N - 1;
      src[h] = D + l * plane + n * ldd + 16 * c;
    }
    off[h] = 1024 * g;
  }
  const int mine = (INS - wave + NW - 1) / NW;  // loads this wave issues per stage (uniform)
  auto issue = [&](int64_t kstep, int buf) {
    int8_t* base = smem + buf * STAGE_BYTES;
    const int64_t k0 = kstep * TKB;
#pragma unroll
    for (int h = 0; h < DMA_MAX; ++h)
      if (h < mine) pipe::dma16(src[h] + k0, base + off[h]);
  };

  v16i acc[2][NL];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int l = 0; l < NL; ++l) acc[i][l] = (v16i){};

  // LDS byte offsets of this lane's operand reads (K half ks adds 32 bytes before swizzling)
  const int ar0 = wm * 64 + (lane & 31), br0 = wn * 32 + (lane & 31);
  const int hs = lane >> 5;

  const int nk = (int)((K + TKB - 1) / TKB);
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, st);
  int cur = 0;  // buffer of step t; step t + STAGES - 1 goes into the one before it
  for (int t = 0; t < nk; ++t) {
    const int ahead = min(STAGES - 2, nk - 1 - t);
    if (mine == DMA_MAX)
      pipe::wait_ahead<DMA_MAX, STAGES - 2>(ahead);
    else
      pipe::wait_ahead<(DMA_MAX > 1 ? DMA_MAX - 1 : 1), STAGES - 2>(ahead);
    pipe::barrier_lds();  // step t is in LDS for every wave; every wave is done with step t - 1
    if (t + STAGES - 1 < nk) issue(t + STAGES - 1, cur == 0 ? STAGES - 1 : cur - 1);
    const int8_t* As = smem + cur * STAGE_BYTES;
    cur = (cur == STAGES - 1) ? 0 : cur + 1;
    const int8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < TKB / 32; ++ks) {
      const int c = 2 * ks + hs;
      v4i a[2], b[NL];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = ar0 + 32 * i;
        a[i] = *reinterpret_cast<const v4i*>(As + r * TKB + 16 * (c ^ swz(r)));
      }
#pragma unroll
      for (int l = 0; l < NL; ++l)
        b[l] = *reinterpret_cast<const v4i*>(Bs + l * TN * TKB + br0 * TKB + 16 * (c ^ swz(br0)));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int l = 0; l < NL; ++l)
          acc[i][l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[l], acc[i][l], 0, 0, 0);
    }
  }

  if (!Cfg::C_FIRST && beta != 0.0) load_c();
  if (!ncol_ok) return;
  const double es = escale[ncol];
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
        C[m * ldc + ncol] = (beta != 0.0) ? fma(beta, cold[i][r], f) : f;
      }
    }
}

using I8Small = I8Tile<128, 4>;
using I8Large = I8Tile<256, 8>;
constexpr int64_t I8_LARGE_MIN_TILES = 256;  // the CU count of the chip

}  // namespace

int launch_limb_pack(const double* U, int64_t ldu, int64_t n, const double* invd, double* escale,
                     double* bscale, int8_t* D, int64_t ldd, hipStream_t st) {
  WSIC_LAUNCH("limb_scale", 8.0 * n * n / 2, st, k_row_scale, dim3((unsigned)n), dim3(256), 0, U,
              ldu, n, invd, escale, bscale);
  if (ldd % 4 != 0 || (((uintptr_t)D) & 3) != 0) {
    set_error("internal: digit plane layout");
    return WSIC_E_INVAL;
  }
  WSIC_LAUNCH("limb_digits", (double)n * ldd * (4.0 + NL), st, k_limb_digits,
              dim3((unsigned)((ldd / 4 + 255) / 256), (unsigned)n), dim3(256), 0, U, ldu, n, invd,
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
  // whole 64-column K-steps are read: the caller's buffers must extend (zero) that far
  if (K % TKB != 0 && (lda < K + (TKB - K % TKB) || ldd < K + (TKB - K % TKB))) {
    set_error("internal: int8 operands shorter than whole K-steps");
    return WSIC_E_INVAL;
  }
  const int64_t tiles_n = (N + TN - 1) / TN;
  // algorithmic int8 ops: NL digit products per multiply-add
  const double work = 2.0 * NL * (double)M * (double)N * (double)K;
  // the large tile when it still gives every CU a workgroup
  const int64_t tiles_large = ((M + I8Large::TM - 1) / I8Large::TM) * tiles_n;
  if (tiles_large >= I8_LARGE_MIN_TILES) {
    WSIC_LAUNCH("gemm_trail_i8", work, st, k_gemm_i8<I8Large>, dim3((unsigned)tiles_large),
                dim3(64 * I8Large::NW), 0, M, N, K, A8, lda, D, ldd, plane, escale, C, ldc, beta,
                (int)tiles_n);
  } else {
    const int64_t tiles = ((M + I8Small::TM - 1) / I8Small::TM) * tiles_n;
    WSIC_LAUNCH("gemm_trail_i8", work, st, k_gemm_i8<I8Small>, dim3((unsigned)tiles),
                dim3(64 * I8Small::NW), 0, M, N, K, A8, lda, D, ldd, plane, escale, C, ldc, beta,
                (int)tiles_n);
  }
  return WSIC_OK;
}

}  // namespace wsic
