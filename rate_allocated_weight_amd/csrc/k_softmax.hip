// Softmax curvature of a classification layer (SoftWater page, §2 "Aproximação Tratável":
// lambda_bar_k = E[p_k (1 - p_k)] over the calibration inputs, p = softmax(W x); §2 "Prior de
// Suavização": p mixed with the uniform distribution over the K classes, weight eps).
//
//   k_logits_bf16     logits L = X W^T (rows x K) on bf16 MFMA, fp32 sums, written as fp32;
//                     per row and 128-class tile the pair (max, sum exp(l - max))
//   k_logits_generic  the same for f32 inputs or shapes the MFMA kernel does not take (fp64 sums)
//   k_softmax_rows    per row: max and 1 / sum exp(l - max) from the tile pairs
//   k_curvature       streams L once: p~ = (1 - eps) p + eps / K, sums p~ (1 - p~) in fp64 over
//                     a chunk of rows per class
//   k_curv_reduce     lambda_k <- beta lambda_k + alpha * (sum of the chunks, fixed order)
//
// Row scales for the class-aware grids (s_k = sqrt(lambda_k)) and their use on Y = W U^T:
//   k_row_sqrt, k_scale_rows.
#include "common.h"
#include "pipe.h"

namespace wsic {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int LT = 128;                 // tile: 128 rows of X x 128 classes
constexpr int LK = 64;                  // K-step in bf16 elements (128 bytes of a row)
constexpr int STRIP = LT * LK * 2;      // 16 KiB
constexpr int STAGE = 2 * STRIP;        // X strip + W strip
constexpr int INS = STRIP / 1024 / 4;   // direct loads per wave per strip
constexpr int CURV_ROWS = 64;           // rows per curvature chunk

__device__ __forceinline__ double ld_elem(const float* p, int64_t i) { return (double)p[i]; }
__device__ __forceinline__ double ld_elem(const uint16_t* p, int64_t i) {
  return (double)__uint_as_float((uint32_t)p[i] << 16);
}

// bf16 logits, 4 waves in 2 x 2, each 64 x 64 = 2 x 2 fragments of v_mfma_f32_32x32x16_bf16.
// Per K-step the two 128 x 64 strips (rows of X, rows of W) go global -> LDS directly, in their
// own row-major layout with the 16-byte chunks of row r XOR-swizzled by r & 7, so an operand
// read of 32 rows x 16 bytes touches every bank once. Two stages in separate LDS objects: the
// loads into one are in flight while the other is read, and the compiler orders no read behind
// them. Operands come through buffer resources, so rows, classes and columns past the matrices
// read zeros. Grid: x = row tile (fastest: the 8 XCDs each hold the same W strip in L2),
// y = class tile. Requirements (launcher): n, ldx, ldw multiples of 8, 16-byte aligned
// operands, both spans below 2 GiB.
__global__ __launch_bounds__(256, 2) void k_logits_bf16(const uint16_t* __restrict__ X, int64_t rows,
                                                        int64_t n, int64_t ldx,
                                                        const uint16_t* __restrict__ W, int64_t K,
                                                        int64_t ldw, float* __restrict__ Lg,
                                                        int64_t ldl, float2* __restrict__ part,
                                                        int ntn) {
  __shared__ __attribute__((aligned(1024))) char SA[STAGE];
  __shared__ __attribute__((aligned(1024))) char SB[STAGE];
  __shared__ float2 xch[2][LT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * LT, c0 = (int64_t)blockIdx.y * LT;
  const int wm = wave >> 1, wn = wave & 1;

  // direct loads: instruction h of this wave fills rows 8 (INS wave + h) + lane / 8 of a strip,
  // 16-byte slot lane % 8, which holds the row's chunk (lane % 8) ^ (row % 8)
  const int chunk = (lane & 7) ^ (lane >> 3);
  int64_t arow[INS], brow[INS];
#pragma unroll
  for (int h = 0; h < INS; ++h) {
    const int r = 8 * (INS * wave + h) + (lane >> 3);
    arow[h] = i0 + r < rows ? (i0 + r) * ldx : -1;
    brow[h] = c0 + r < K ? (c0 + r) * ldw : -1;
  }
  const __amdgpu_buffer_rsrc_t xr = pipe::make_rsrc(X, (unsigned)(rows * ldx * 2));
  const __amdgpu_buffer_rsrc_t wr = pipe::make_rsrc(W, (unsigned)(K * ldw * 2));
  auto issue = [&](int64_t k0, char* S) {
    const int64_t col = k0 + 8 * chunk;
    const bool cok = col < n;
#pragma unroll
    for (int h = 0; h < INS; ++h) {
      const unsigned va = (cok && arow[h] >= 0) ? (unsigned)((arow[h] + col) * 2) : pipe::OUT_OF_RANGE;
      const unsigned vb = (cok && brow[h] >= 0) ? (unsigned)((brow[h] + col) * 2) : pipe::OUT_OF_RANGE;
      pipe::dma16_buf(xr, va, S + 1024 * (INS * wave + h));
      pipe::dma16_buf(wr, vb, S + STRIP + 1024 * (INS * wave + h));
    }
  };

  f16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f16v){};

  const int half = lane >> 5, l32 = lane & 31;
  auto compute = [&](const char* S) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < LK / 16; ++ks) {
      const int ch = 2 * ks + half;
      bf8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + l32;
        const uint4 v = *reinterpret_cast<const uint4*>(S + r * 128 + 16 * (ch ^ (r & 7)));
        __builtin_memcpy(&a[i], &v, 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + 32 * j + l32;
        const uint4 v = *reinterpret_cast<const uint4*>(S + STRIP + r * 128 + 16 * (ch ^ (r & 7)));
        __builtin_memcpy(&b[j], &v, 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // step t: its loads (the only ones in flight) land, every wave is past step t - 1 (whose
  // buffer is refilled now), then the next step's loads go out and this one is computed
  const int nk = (int)((n + LK - 1) / LK);
  issue(0, SA);
  for (int t = 0; t < nk; t += 2) {
    pipe::wait_vm<0>();
    pipe::barrier_lds();
    if (t + 1 < nk) issue((int64_t)(t + 1) * LK, SB);
    compute(SA);
    if (t + 1 < nk) {
      pipe::wait_vm<0>();
      pipe::barrier_lds();
      if (t + 2 < nk) issue((int64_t)(t + 2) * LK, SA);
      compute(SB);
    }
  }

  // logits and the per-row (max, sum exp) of this tile's classes
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rt = wm * 64 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);  // row in the tile
      const int64_t row = i0 + rt;
      float v[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = c0 + wn * 64 + 32 * j + l32;
        const bool ok = col < K;
        v[j] = ok ? acc[i][j][r] : -INFINITY;
        if (ok && row < rows) Lg[row * ldl + col] = acc[i][j][r];
      }
      float m = fmaxf(v[0], v[1]);
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      float s = (m == -INFINITY) ? 0.0f : expf(v[0] - m) + expf(v[1] - m);
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) s += __shfl_xor(s, d, 64);
      if (l32 == 0) xch[wn][rt] = make_float2(m, s);
    }
  }
  __syncthreads();
  if (tid < LT && i0 + tid < rows) {
    const float2 a = xch[0][tid], b = xch[1][tid];
    const float m = fmaxf(a.x, b.x);
    const float s = (a.x == -INFINITY ? 0.0f : a.y * expf(a.x - m)) +
                    (b.x == -INFINITY ? 0.0f : b.y * expf(b.x - m));
    part[(i0 + tid) * ntn + blockIdx.y] = make_float2(m, s);
  }
}

// Any dtype and shape: one thread per (row, class), fp64 sums.
template <typename T>
__global__ __launch_bounds__(LT) void k_logits_generic(const T* __restrict__ X, int64_t rows,
                                                       int64_t n, int64_t ldx,
                                                       const T* __restrict__ W, int64_t K,
                                                       int64_t ldw, float* __restrict__ Lg,
                                                       int64_t ldl, float2* __restrict__ part,
                                                       int ntn) {
  __shared__ float sm[LT], ss[LT];
  const int64_t row = blockIdx.y;
  const int64_t k = (int64_t)blockIdx.x * LT + threadIdx.x;
  float v = -INFINITY;
  if (k < K) {
    double a = 0.0;
    for (int64_t i = 0; i < n; ++i)
      a = fma(ld_elem(X, row * ldx + i), ld_elem(W, k * ldw + i), a);
    v = (float)a;
    Lg[row * ldl + k] = v;
  }
  sm[threadIdx.x] = v;
  __syncthreads();
  for (int d = LT / 2; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) sm[threadIdx.x] = fmaxf(sm[threadIdx.x], sm[threadIdx.x + d]);
    __syncthreads();
  }
  const float m = sm[0];
  ss[threadIdx.x] = (k < K) ? expf(v - m) : 0.0f;
  __syncthreads();
  for (int d = LT / 2; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) ss[threadIdx.x] += ss[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[row * ntn + blockIdx.x] = make_float2(m, ss[0]);
}

// one wave per row: M = max of the tile maxima, Z = sum_t s_t exp(m_t - M) (Z >= 1)
__global__ __launch_bounds__(256) void k_softmax_rows(const float2* __restrict__ part, int64_t rows,
                                                      int ntn, float* __restrict__ rmax,
                                                      double* __restrict__ rinvz) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float2* p = part + row * ntn;
  float m = -INFINITY;
  for (int t = lane; t < ntn; t += 64) m = fmaxf(m, p[t].x);
  for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  double s = 0.0;
  for (int t = lane; t < ntn; t += 64)
    if (p[t].x != -INFINITY) s += (double)p[t].y * exp((double)p[t].x - (double)m);
  for (int d = 1; d < 64; d <<= 1) s += __shfl_xor(s, d, 64);
  if (lane == 0) {
    rmax[row] = m;
    rinvz[row] = 1.0 / s;
  }
}

// class k per thread, CURV_ROWS rows per chunk; loads of one row are contiguous across threads
__global__ __launch_bounds__(256) void k_curvature(const float* __restrict__ Lg, int64_t ldl,
                                                   int64_t rows, int64_t K,
                                                   const float* __restrict__ rmax,
                                                   const double* __restrict__ rinvz, double eps,
                                                   double* __restrict__ cpart) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * CURV_ROWS;
  const int64_t r1 = r0 + CURV_ROWS < rows ? r0 + CURV_ROWS : rows;
  if (k >= K) return;
  const double u = eps / (double)K, keep = 1.0 - eps;
  double acc = 0.0;
#pragma unroll 4
  for (int64_t r = r0; r < r1; ++r) {
    const double p = (double)expf(Lg[r * ldl + k] - rmax[r]) * rinvz[r];
    const double pt = fma(keep, p, u);
    acc = fma(pt, 1.0 - pt, acc);
  }
  cpart[(int64_t)blockIdx.y * K + k] = acc;
}

__global__ void k_curv_reduce(const double* __restrict__ cpart, int nchunk, int64_t K,
                              double alpha, double beta, double* __restrict__ lam,
                              int* __restrict__ flags) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  double s = 0.0;
  for (int c = 0; c < nchunk; ++c) s += cpart[(int64_t)c * K + k];
  const double v = (beta != 0.0) ? fma(alpha, s, beta * lam[k]) : alpha * s;
  if (!isfinite(v)) atomicOr(flags, FLAG_NONFINITE);
  lam[k] = v;
}

__global__ void k_row_sqrt(const double* __restrict__ lam, int64_t n, double* __restrict__ s,
                           int* __restrict__ flags) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const double v = lam[k];
  if (!(v > 0.0) || !isfinite(v)) {
    atomicOr(flags, FLAG_BAD_SCALE);
    s[k] = 1.0;
  } else {
    s[k] = sqrt(v);
  }
}

__global__ void k_scale_rows(double* __restrict__ Y, int64_t n_out, int64_t n_in, int64_t ldy,
                             const double* __restrict__ s) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (j < n_in) Y[r * ldy + j] *= s[r];
}

}  // namespace

void curvature_dims(int64_t rows, int64_t K, int64_t* ntn, int64_t* nchunk, int64_t* ldl) {
  *ntn = (K + LT - 1) / LT;
  *nchunk = (rows + CURV_ROWS - 1) / CURV_ROWS;
  *ldl = (K + 63) / 64 * 64;
}

int launch_softmax_curvature(const CurvArgs& a, hipStream_t st) {
  const int64_t ntn = (a.K + LT - 1) / LT;
  const int64_t ntm = (a.rows + LT - 1) / LT;
  const int64_t nchunk = (a.rows + CURV_ROWS - 1) / CURV_ROWS;
  if (ntn > 65535 || a.rows > 65535 * (int64_t)CURV_ROWS ||
      (a.rows > 65535 && !(a.dtype == WSIC_BF16 && !a.force_generic))) {
    set_error("softmax_curvature: too many classes or rows in one call (split the rows)");
    return WSIC_E_INVAL;
  }
  const bool mfma = a.dtype == WSIC_BF16 && a.n % 8 == 0 && a.ldx % 8 == 0 && a.ldw % 8 == 0 &&
                    ((uintptr_t)a.X & 15) == 0 && ((uintptr_t)a.W & 15) == 0 &&
                    a.rows * a.ldx * 2 < (int64_t)pipe::OUT_OF_RANGE &&
                    a.K * a.ldw * 2 < (int64_t)pipe::OUT_OF_RANGE && !a.force_generic;
  const double flops = 2.0 * (double)a.rows * (double)a.K * (double)a.n;
  if (mfma) {
    WSIC_LAUNCH("logits_bf16", flops, st, k_logits_bf16, dim3((unsigned)ntm, (unsigned)ntn),
                dim3(256), 0, (const uint16_t*)a.X, a.rows, a.n, a.ldx, (const uint16_t*)a.W, a.K,
                a.ldw, a.Lg, a.ldl, a.part, (int)ntn);
  } else if (a.dtype == WSIC_BF16) {
    WSIC_LAUNCH("logits_generic", flops, st, k_logits_generic<uint16_t>,
                dim3((unsigned)ntn, (unsigned)a.rows), dim3(LT), 0, (const uint16_t*)a.X, a.rows,
                a.n, a.ldx, (const uint16_t*)a.W, a.K, a.ldw, a.Lg, a.ldl, a.part, (int)ntn);
  } else {
    WSIC_LAUNCH("logits_generic", flops, st, k_logits_generic<float>,
                dim3((unsigned)ntn, (unsigned)a.rows), dim3(LT), 0, (const float*)a.X, a.rows, a.n,
                a.ldx, (const float*)a.W, a.K, a.ldw, a.Lg, a.ldl, a.part, (int)ntn);
  }
  WSIC_LAUNCH("softmax_rows", 8.0 * (double)a.rows * ntn, st, k_softmax_rows,
              dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, a.part, a.rows, (int)ntn, a.rmax,
              a.rinvz);
  WSIC_LAUNCH("curvature", 4.0 * (double)a.rows * a.K + 8.0 * (double)nchunk * a.K, st,
              k_curvature, dim3((unsigned)((a.K + 255) / 256), (unsigned)nchunk), dim3(256), 0,
              a.Lg, a.ldl, a.rows, a.K, a.rmax, a.rinvz, a.eps, a.cpart);
  WSIC_LAUNCH("curv_reduce", 8.0 * (double)nchunk * a.K, st, k_curv_reduce,
              dim3((unsigned)((a.K + 255) / 256)), dim3(256), 0, a.cpart, (int)nchunk, a.K, a.alpha,
              a.beta, a.lam, a.flags);
  return WSIC_OK;
}

int launch_row_sqrt(const double* lam, int64_t n, double* s, int* flags, hipStream_t st) {
  WSIC_LAUNCH("row_scale", 16.0 * n, st, k_row_sqrt, dim3((unsigned)((n + 255) / 256)), dim3(256),
              0, lam, n, s, flags);
  return WSIC_OK;
}

int launch_scale_rows(double* Y, int64_t n_out, int64_t n_in, int64_t ldy, const double* s,
                      hipStream_t st) {
  if (n_out > 65535) {
    // rows in slices of 65535 (grid y limit)
    for (int64_t r0 = 0; r0 < n_out; r0 += 65535) {
      const int64_t nr = n_out - r0 < 65535 ? n_out - r0 : 65535;
      const int rc = launch_scale_rows(Y + r0 * ldy, nr, n_in, ldy, s + r0, st);
      if (rc != WSIC_OK) return rc;
    }
    return WSIC_OK;
  }
  WSIC_LAUNCH("scale_rows", 16.0 * (double)n_out * n_in, st, k_scale_rows,
              dim3((unsigned)((n_in + 255) / 256), (unsigned)n_out), dim3(256), 0, Y, n_out, n_in,
              ldy, s);
  return WSIC_OK;
}

}  // namespace wsic
