// Per-column code entropy and the Gaussian rate-distortion limit (WaterSIC page, §3 Limiti teorici:
// WaterSIC is within 1/2 log2(2 pi e / 12) bit of the information-theoretic limit, a reverse
// waterfilling, when each input column is entropy coded on its own step; §2 item 3: the codes are
// unbounded integers).
//
//   k_hist_cols    column histograms: a workgroup takes 32 columns x 512 rows; each thread walks
//                  one column, tallying codes in [-7, 8] in 16-bit register counters (two per
//                  register), summed over the two threads of the same column in a wave; other
//                  codes within +-127 go to an LDS window per column, wider ones to an overflow
//                  list (column, code) that the host counts exactly
//   k_col_entropy  S_j = sum_k n_jk log2 n_jk per column (fp64)
//   k_sumsq        partial sums of w^2 (the weight variance of the Gaussian model)
//   k_logdiag      partial sums of log2 U_jj (det Sigma = prod U_jj^2)
#include "common.h"

namespace wsic {
namespace {

constexpr int CREG_LO = -7, CREG_N = 16;

__global__ __launch_bounds__(256) void k_hist_cols(const int32_t* __restrict__ codes, int64_t n_out,
                                                   int64_t n_in, int64_t ldq,
                                                   unsigned* __restrict__ colbins,
                                                   int2* __restrict__ ovf,
                                                   unsigned* __restrict__ ovf_count) {
  __shared__ unsigned h[COL_TILE * COL_BINS];
  const int tid = threadIdx.x;
  for (int i = tid; i < COL_TILE * COL_BINS; i += 256) h[i] = 0u;
  __syncthreads();
  const int c = tid & (COL_TILE - 1), rl = tid / COL_TILE;  // 8 row lanes
  const int64_t j = (int64_t)blockIdx.x * COL_TILE + c;
  const int64_t r0 = (int64_t)blockIdx.y * COL_ROWS;
  const int64_t r1 = r0 + COL_ROWS < n_out ? r0 + COL_ROWS : n_out;
  unsigned reg[CREG_N / 2];
#pragma unroll
  for (int k = 0; k < CREG_N / 2; ++k) reg[k] = 0u;
  if (j < n_in) {
    for (int64_t r = r0 + rl; r < r1; r += 256 / COL_TILE) {
      const int v = codes[r * ldq + j];
      const int t = v - CREG_LO;
      if (t >= 0 && t < CREG_N) {
        const unsigned inc = 1u << (16 * (t & 1));
#pragma unroll
        for (int k = 0; k < CREG_N / 2; ++k) reg[k] += ((t >> 1) == k) ? inc : 0u;
      } else if (v >= -COL_HALF && v <= COL_HALF) {
        atomicAdd(&h[c * COL_BINS + v + COL_HALF], 1u);
      } else {
        const unsigned slot = atomicAdd(ovf_count, 1u);
        if (slot < OVF_CAP) ovf[slot] = make_int2((int)j, v);
      }
    }
  }
  // the two threads of a column in a wave (lanes c and c + 32) hold at most 2 x 64 codes each
  // bin: the 16-bit counters cannot carry
#pragma unroll
  for (int k = 0; k < CREG_N / 2; ++k) reg[k] += __shfl_xor(reg[k], COL_TILE, 64);
  if ((tid & 63) < COL_TILE && j < n_in) {
#pragma unroll
    for (int k = 0; k < CREG_N / 2; ++k) {
      const unsigned lo = reg[k] & 0xffffu, hi = reg[k] >> 16;
      if (lo) atomicAdd(&h[c * COL_BINS + (CREG_LO + 2 * k) + COL_HALF], lo);
      if (hi) atomicAdd(&h[c * COL_BINS + (CREG_LO + 2 * k + 1) + COL_HALF], hi);
    }
  }
  __syncthreads();
  for (int i = tid; i < COL_TILE * COL_BINS; i += 256) {
    const unsigned n = h[i];
    const int64_t jj = (int64_t)blockIdx.x * COL_TILE + i / COL_BINS;
    if (n && jj < n_in) atomicAdd(&colbins[jj * COL_BINS + i % COL_BINS], n);
  }
}

__global__ void k_col_entropy(const unsigned* __restrict__ colbins, int64_t n_in,
                              double* __restrict__ colS) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_in) return;
  double s = 0.0;
  for (int b = 0; b < COL_BINS; ++b) {
    const unsigned n = colbins[j * COL_BINS + b];
    if (n > 1u) s += (double)n * log2((double)n);
  }
  colS[j] = s;
}

template <typename T>
__device__ __forceinline__ double ld_w(const T* p, int64_t i);
template <>
__device__ __forceinline__ double ld_w<float>(const float* p, int64_t i) {
  return (double)p[i];
}
template <>
__device__ __forceinline__ double ld_w<uint16_t>(const uint16_t* p, int64_t i) {
  return (double)__uint_as_float((uint32_t)p[i] << 16);
}

template <typename T>
__global__ __launch_bounds__(256) void k_sumsq(const T* __restrict__ W, int64_t n_out, int64_t n_in,
                                               int64_t ldw, double* __restrict__ partial) {
  __shared__ double red[256];
  double s = 0.0;
  const int64_t total = n_out * n_in;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / n_in, j = e - r * n_in;
    const double v = ld_w<T>(W, r * ldw + j);
    s = fma(v, v, s);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int d = 128; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ void k_logdiag(const double* __restrict__ U, int64_t ldu, int64_t n,
                          double* __restrict__ out, int* __restrict__ flags) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const double d = U[j * ldu + j];
  if (!(d > 0.0) || !isfinite(d)) atomicOr(flags, FLAG_BAD_DIAG);
  out[j] = log2(d > 0.0 ? d : 1.0);
}

}  // namespace

int launch_hist_cols(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                     unsigned* colbins, int2* ovf, unsigned* ovf_count, hipStream_t st) {
  const int64_t gx = (n_in + COL_TILE - 1) / COL_TILE, gy = (n_out + COL_ROWS - 1) / COL_ROWS;
  if (gx > 0x7fffffff || gy > 65535) {
    set_error("entropy_columns: %lld rows exceed the grid", (long long)n_out);
    return WSIC_E_INVAL;
  }
  WSIC_LAUNCH("hist_cols", 4.0 * (double)n_out * n_in, st, k_hist_cols, dim3((unsigned)gx, (unsigned)gy),
              dim3(256), 0, codes, n_out, n_in, ldq, colbins, ovf, ovf_count);
  return WSIC_OK;
}

int launch_col_entropy(const unsigned* colbins, int64_t n_in, double* colS, hipStream_t st) {
  WSIC_LAUNCH("col_entropy", 4.0 * (double)n_in * COL_BINS, st, k_col_entropy,
              dim3((unsigned)((n_in + 255) / 256)), dim3(256), 0, colbins, n_in, colS);
  return WSIC_OK;
}

int launch_sumsq(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw, double* partial,
                 int nblk, hipStream_t st) {
  const double work = (double)n_out * n_in * (dtype == WSIC_BF16 ? 2.0 : 4.0);
  if (dtype == WSIC_BF16)
    WSIC_LAUNCH("sumsq", work, st, k_sumsq<uint16_t>, dim3((unsigned)nblk), dim3(256), 0,
                (const uint16_t*)W, n_out, n_in, ldw, partial);
  else
    WSIC_LAUNCH("sumsq", work, st, k_sumsq<float>, dim3((unsigned)nblk), dim3(256), 0, (const float*)W,
                n_out, n_in, ldw, partial);
  return WSIC_OK;
}

int launch_logdiag(const double* U, int64_t ldu, int64_t n, double* out, int* flags, hipStream_t st) {
  WSIC_LAUNCH("logdiag", 16.0 * n, st, k_logdiag, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, U,
              ldu, n, out, flags);
  return WSIC_OK;
}

}  // namespace wsic
