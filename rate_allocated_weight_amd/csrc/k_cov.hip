// Calibration covariance Sigma = beta Sigma + alpha X^T X (SYRK; WaterSIC page, Sommario
// tecnico §2 item 1, where the covariance of the input activations is factorized).
//
// bf16 X: v_mfma_f32_32x32x16_bf16. bf16 x bf16 products are exact in fp32; a K-step of 64
// calibration rows is summed in fp32 by the MFMAs and then folded into fp64 accumulators, so
// rounding error does not grow with the number of rows. Tile 64 x 64 of Sigma per 256-thread
// workgroup (4 waves, one 32 x 32 MFMA tile each), upper-triangle tiles only.
// X is row-major (rows x n), i.e. k-major for this product; the MFMA wants 8 consecutive k
// per lane, so each loading thread reads an 8 x 8 block of X (8 rows x 16 bytes), transposes
// it in registers and writes 8 k-contiguous 16-byte rows to LDS.
//
// f32 X: products and sums in fp64 on the vector ALUs (the small workloads that use fp32
// calibration data do not need matrix cores).
//
// MFMA 32x32x16 bf16 lane layout (checked on gfx950): A operand lane l holds
// A[l%32][8*(l/32) + e], B operand B[8*(l/32) + e][l%32], result register r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "common.h"
#include "pipe.h"

namespace wsic {
namespace {

constexpr int T = 64;    // Sigma tile
constexpr int TKR = 64;  // calibration rows per K-step
constexpr int LROW = TKR + 8;  // LDS row length (bf16 elements), 144 bytes

typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

struct U4 {
  uint32_t w[4];
};

// 8 bf16 of row r starting at column c; zero outside [0,rows) x [0,n)
__device__ __forceinline__ U4 load8(const uint16_t* X, int64_t ldx, int64_t rows, int64_t n,
                                    int64_t r, int64_t c, bool vec_ok) {
  U4 v;
  if (r < rows && c + 8 <= n && vec_ok) {
    const uint4 t = *reinterpret_cast<const uint4*>(X + r * ldx + c);
    v.w[0] = t.x;
    v.w[1] = t.y;
    v.w[2] = t.z;
    v.w[3] = t.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo = 0, hi = 0;
      if (r < rows && c + 2 * q < n) lo = X[r * ldx + c + 2 * q];
      if (r < rows && c + 2 * q + 1 < n) hi = X[r * ldx + c + 2 * q + 1];
      v.w[q] = lo | (hi << 16);
    }
  }
  return v;
}

__device__ __forceinline__ uint32_t half_of(uint32_t w, int h) { return h ? (w >> 16) : (w & 0xffffu); }

__global__ __launch_bounds__(256) void k_syrk_bf16(const uint16_t* __restrict__ X, int64_t rows,
                                                   int64_t n, int64_t ldx, double alpha,
                                                   double beta, double* __restrict__ S,
                                                   int64_t lds, int tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t As[T][LROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[T][LROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ti = blockIdx.x / tiles, tj = blockIdx.x % tiles;
  if (tj < ti) return;
  const int64_t i0 = (int64_t)ti * T, j0 = (int64_t)tj * T;
  const bool vec_ok = ((ldx & 7) == 0) && ((((uintptr_t)X) & 15) == 0);

  // loader: threads 0..63 fill As, 64..127 fill Bs; 8 x 8 block (br, bc)
  const bool loader = tid < 128;
  const int lt = tid & 63;
  const int br = lt >> 3, bc = lt & 7;
  const int64_t col0 = (tid < 64 ? i0 : j0) + 8 * bc;
  uint16_t(*dst)[LROW] = (tid < 64) ? As : Bs;

  const int wm = wave >> 1, wn = wave & 1;
  double acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0;

  for (int64_t r0 = 0; r0 < rows; r0 += TKR) {
    if (loader) {
      U4 R[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) R[e] = load8(X, ldx, rows, n, r0 + 8 * br + e, col0, vec_ok);
      // transpose: output column c gathers element c of the 8 rows
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint4 o;
        uint32_t ow[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ow[q] = half_of(R[2 * q].w[c >> 1], c & 1) | (half_of(R[2 * q + 1].w[c >> 1], c & 1) << 16);
        o.x = ow[0];
        o.y = ow[1];
        o.z = ow[2];
        o.w = ow[3];
        *reinterpret_cast<uint4*>(&dst[8 * bc + c][8 * br]) = o;
      }
    }
    __syncthreads();
    f16v p = {};
#pragma unroll
    for (int ks = 0; ks < TKR / 16; ++ks) {
      const uint4 av = *reinterpret_cast<const uint4*>(&As[wm * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
      const uint4 bv = *reinterpret_cast<const uint4*>(&Bs[wn * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
      bf8 a, b;
      __builtin_memcpy(&a, &av, 16);
      __builtin_memcpy(&b, &bv, 16);
      p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, p, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += (double)p[r];
    __syncthreads();
  }

#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t i = i0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int64_t j = j0 + wn * 32 + (lane & 31);
    if (i < n && j < n && j >= i) {
      double* p = S + i * lds + j;
      *p = (beta != 0.0) ? fma(alpha, acc[r], beta * *p) : alpha * acc[r];
    }
  }
}

// bf16 X, pipelined: Sigma tile 128 x 128 per 256-thread workgroup (upper tiles only, enumerated
// triangularly); 4 waves in 2 x 2, each 64 x 64 = 2 x 2 fragments of v_mfma_f32_32x32x16_bf16.
// Per K-step of 128 calibration rows the two 128 x 128 row strips of X (the tile's rows and its
// columns of Sigma) go global -> LDS directly (global_load_lds_dwordx4) through a ring of 2
// buffers, in X's own row-major layout with the 16-byte chunks of row r XOR-swizzled by 2 (r & 3).
// The MFMA wants 8 consecutive rows of X per lane; ds_read_b64_tr_b16 delivers them: within each
// 16-lane group, lane i receives element i % 4 of the 8-byte rows addressed by lanes 4v + i / 4
// (v = 0..3, checked on gfx950), so lanes pointing at [k0 + j/4][c0 + 4 (j%4)] hand lane i the
// values X[k0 .. k0+3][c0 + i]. fp32 sums over 256 rows are folded into fp64 accumulators.
// Operands are read through a buffer resource over X, so rows and columns past the matrix read
// zeros. Requirements (checked by the launcher): n % 8 == 0, ldx % 8 == 0, X 16-byte aligned,
// X's span below 2 GiB.
namespace sdma {
constexpr int T = 128, TKR = 128, STAGES = 2, FOLD_STEPS = 256 / TKR;
constexpr int STRIP = TKR * T * 2;  // 32 KiB: 128 rows x 128 bf16
constexpr int STAGE = 2 * STRIP;
constexpr int INS = STRIP / 4096;   // DMA instructions per wave per strip
constexpr int DMA = 2 * INS;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
// byte offset of bf16 column c of row r inside a strip
__device__ __forceinline__ int strip_off(int r, int c) {
  return r * (T * 2) + (((c >> 3) ^ (2 * (r & 3))) << 4) + ((c & 7) << 1);
}
}  // namespace sdma

__global__ __launch_bounds__(256) void k_syrk_bf16_dma(const uint16_t* __restrict__ X, int64_t rows,
                                                       int64_t n, int64_t ldx, double alpha,
                                                       double beta, double* __restrict__ S,
                                                       int64_t lds) {
  constexpr int T = sdma::T, TKR = sdma::TKR, STAGES = sdma::STAGES, FOLD_STEPS = sdma::FOLD_STEPS;
  constexpr int STRIP = sdma::STRIP, STAGE = sdma::STAGE, INS = sdma::INS, DMA = sdma::DMA;
  using sdma::lds_v4s;
  using sdma::v4s;
  using sdma::strip_off;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bid = blockIdx.x;
  int64_t tn = (int64_t)((sqrt(8.0 * (double)bid + 1.0) - 1.0) * 0.5);
  while ((tn + 1) * (tn + 2) / 2 <= bid) ++tn;
  while (tn * (tn + 1) / 2 > bid) --tn;
  const int64_t tm = bid - tn * (tn + 1) / 2;
  const int64_t i0 = tm * T, j0 = tn * T;
  const int wm = wave >> 1, wn = wave & 1;

  // this lane's DMA chunks: strip s, instruction h -> row r, global chunk column col
  int drow[2][INS];
  int64_t dcol[2][INS];
  bool dcol_ok[2][INS];
#pragma unroll
  for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
    for (int h = 0; h < INS; ++h) {
      const int p = 64 * (INS * wave + h) + lane;
      const int r = p >> 4, slot = p & 15;
      const int c = slot ^ (2 * (r & 3));
      drow[sidx][h] = r;
      dcol[sidx][h] = (sidx == 0 ? i0 : j0) + 8 * c;
      dcol_ok[sidx][h] = dcol[sidx][h] < n;
    }
  const __amdgpu_buffer_rsrc_t xr = pipe::make_rsrc(X, (unsigned)(rows * ldx * 2));
  auto issue = [&](int64_t k0, int buf) {
    char* base = smem + buf * STAGE;
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
      for (int h = 0; h < INS; ++h) {
        const int64_t r = k0 + drow[sidx][h];
        const unsigned voff = (r < rows && dcol_ok[sidx][h])
                                  ? (unsigned)((r * ldx + dcol[sidx][h]) * 2)
                                  : pipe::OUT_OF_RANGE;
        pipe::dma16_buf(xr, voff, base + sidx * STRIP + 1024 * (INS * wave + h));
      }
  };

  f16v acc32[2][2];
  double acc64[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc32[i][j] = (f16v){};
#pragma unroll
      for (int r = 0; r < 16; ++r) acc64[i][j][r] = 0.0;
    }

  // operand read coordinates of this lane (16-lane group g, lane j in the group)
  const int g = lane >> 4, jl = lane & 15;
  const int m_off = 16 * (g & 1), k_off = 8 * (g >> 1);
  const int rsub = jl >> 2, csub = 4 * (jl & 3);

  const int nk = (int)((rows + TKR - 1) / TKR);
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue((int64_t)st * TKR, st);
  int cur = 0;
  for (int t = 0; t < nk; ++t) {
    pipe::wait_ahead<DMA, STAGES - 2>(min(STAGES - 2, nk - 1 - t));
    pipe::barrier_lds();
    if (t + STAGES - 1 < nk) issue((int64_t)(t + STAGES - 1) * TKR, cur == 0 ? STAGES - 1 : cur - 1);
    const char* As = smem + cur * STAGE;
    const char* Bs = As + STRIP;
    cur = (cur == STAGES - 1) ? 0 : cur + 1;
#pragma unroll
    for (int ks = 0; ks < TKR / 16; ++ks) {
      bf8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int cbase = wm * 64 + i * 32 + m_off + csub;
        v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(As + strip_off(ks * 16 + k_off + rsub, cbase)));
        v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(As + strip_off(ks * 16 + k_off + 4 + rsub, cbase)));
        short e8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        __builtin_memcpy(&a[i], e8, 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cbase = wn * 64 + j * 32 + m_off + csub;
        v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(Bs + strip_off(ks * 16 + k_off + rsub, cbase)));
        v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(Bs + strip_off(ks * 16 + k_off + 4 + rsub, cbase)));
        short e8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        __builtin_memcpy(&b[j], e8, 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc32[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc32[i][j], 0, 0, 0);
    }
    if ((t + 1) % FOLD_STEPS == 0 || t + 1 == nk) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc64[i][j][r] += (double)acc32[i][j][r];
          acc32[i][j] = (f16v){};
        }
    }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t ii = i0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t jj = j0 + wn * 64 + j * 32 + (lane & 31);
        if (ii < n && jj < n && jj >= ii) {
          double* p = S + ii * lds + jj;
          *p = (beta != 0.0) ? fma(alpha, acc64[i][j][r], beta * *p) : alpha * acc64[i][j][r];
        }
      }
}

__global__ __launch_bounds__(256) void k_syrk_f32(const float* __restrict__ X, int64_t rows,
                                                  int64_t n, int64_t ldx, double alpha, double beta,
                                                  double* __restrict__ S, int64_t lds, int tiles) {
  constexpr int TK = 16;
  __shared__ double Xa[TK][T + 1];
  __shared__ double Xb[TK][T + 1];
  const int tid = threadIdx.x;
  const int ti = blockIdx.x / tiles, tj = blockIdx.x % tiles;
  if (tj < ti) return;
  const int64_t i0 = (int64_t)ti * T, j0 = (int64_t)tj * T;
  const int tx = tid & 15, ty = tid >> 4;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t r0 = 0; r0 < rows; r0 += TK) {
    for (int e = tid; e < TK * T; e += 256) {
      const int k = e / T, c = e % T;
      const int64_t r = r0 + k;
      Xa[k][c] = (r < rows && i0 + c < n) ? (double)X[r * ldx + i0 + c] : 0.0;
      Xb[k][c] = (r < rows && j0 + c < n) ? (double)X[r * ldx + j0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = Xa[k][ty * 4 + a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Xb[k][tx * 4 + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t i = i0 + ty * 4 + a, j = j0 + tx * 4 + b;
      if (i < n && j < n && j >= i) {
        double* p = S + i * lds + j;
        *p = (beta != 0.0) ? fma(alpha, acc[a][b], beta * *p) : alpha * acc[a][b];
      }
    }
}

// Copy the strict upper triangle onto the lower one through a 32 x 32 LDS transpose.
__global__ __launch_bounds__(256) void k_mirror(double* S, int64_t n, int64_t lds, int tiles) {
  __shared__ double t[32][33];
  const int bi = blockIdx.x / tiles, bj = blockIdx.x % tiles;  // destination tile (bi >= bj)
  if (bi < bj) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    const int64_t r = (int64_t)bj * 32 + yy, c = (int64_t)bi * 32 + tx;  // source: upper tile
    t[yy][tx] = (r < n && c < n) ? S[r * lds + c] : 0.0;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int64_t r = (int64_t)bi * 32 + yy, c = (int64_t)bj * 32 + tx;  // destination
    if (r < n && c < n && r > c) S[r * lds + c] = t[tx][yy];
  }
}

__global__ void k_diag_check(const double* S, int64_t n, int64_t lds, int* flags) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n && !isfinite(S[j * lds + j])) atomicOr(flags, FLAG_NONFINITE);
}

}  // namespace

int launch_syrk(const void* X, int dtype, int64_t rows, int64_t n, int64_t ldx, double alpha,
                double beta, double* S, int64_t lds, hipStream_t st) {
  const int tiles = (int)((n + T - 1) / T);
  const unsigned grid = (unsigned)((int64_t)tiles * tiles);
  const double work = (double)rows * (double)n * (double)(n + 1);  // flops of the upper triangle
  const bool dma_ok = n % 8 == 0 && ldx % 8 == 0 && (((uintptr_t)X) & 15) == 0 &&
                      rows * ldx * 2 < (int64_t)pipe::OUT_OF_RANGE;
  if (dtype == WSIC_BF16 && dma_ok) {
    const int64_t t = (n + sdma::T - 1) / sdma::T;
    WSIC_LAUNCH("syrk_bf16", work, st, k_syrk_bf16_dma, dim3((unsigned)(t * (t + 1) / 2)), dim3(256),
                0, (const uint16_t*)X, rows, n, ldx, alpha, beta, S, lds);
  } else if (dtype == WSIC_BF16)
    WSIC_LAUNCH("syrk_bf16", work, st, k_syrk_bf16, dim3(grid), dim3(256), 0, (const uint16_t*)X,
                rows, n, ldx, alpha, beta, S, lds, tiles);
  else
    WSIC_LAUNCH("syrk_f32", work, st, k_syrk_f32, dim3(grid), dim3(256), 0, (const float*)X, rows,
                n, ldx, alpha, beta, S, lds, tiles);
  return WSIC_OK;
}

int launch_mirror_upper(double* S, int64_t n, int64_t lds, hipStream_t st) {
  const int tiles = (int)((n + 31) / 32);
  WSIC_LAUNCH("mirror", 8.0 * (double)n * n, st, k_mirror, dim3((unsigned)((int64_t)tiles * tiles)),
              dim3(256), 0, S, n, lds, tiles);
  return WSIC_OK;
}

int launch_diag_check(const double* S, int64_t n, int64_t lds, int* flags, hipStream_t st) {
  WSIC_LAUNCH("diag_check", 8.0 * n, st, k_diag_check, dim3((unsigned)((n + 255) / 256)),
              dim3(256), 0, S, n, lds, flags);
  return WSIC_OK;
}

}  // namespace wsic
