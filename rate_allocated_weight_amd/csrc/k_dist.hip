// Distortion and dequantization passes.
//
// The layer distortion tr((W - W_hat) Sigma (W - W_hat)^T) (the output error of Y = W X,
// WaterSIC page, Sommario tecnico §1) splits per column over the SIC residuals:
//     D = sum_j U_jj^2 sum_i r_ij^2 .
// k_dist_resid streams the fp32 residuals once: a workgroup owns a strip of 1024 columns (four
// per thread, read as 16-byte vectors when the rows allow it) and a slab of DIST_ROWS rows, with
// DIST_UNR rows' loads in flight per thread; each thread keeps its columns' sums of squares in
// fp64, scales them by U_jj^2, and the workgroup writes one partial. Partials are summed in a
// fixed order by k_sum_partials, so the result is deterministic.
#include "common.h"

namespace wsic {
namespace {

constexpr int DIST_COLS = 1024;  // columns per workgroup: 4 per thread
constexpr int DIST_UNR = 8;

__global__ __launch_bounds__(256) void k_dist_resid(const float* __restrict__ resid,
                                                    int64_t n_out, int64_t n_in, int64_t ldr,
                                                    const double* __restrict__ U, int64_t ldu,
                                                    double* __restrict__ partial) {
  __shared__ double red[256];
  const int64_t j = (int64_t)blockIdx.x * DIST_COLS + 4 * threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * DIST_ROWS;
  const int64_t r1 = (r0 + DIST_ROWS < n_out) ? r0 + DIST_ROWS : n_out;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (j + 3 < n_in && (ldr & 3) == 0 && (((uintptr_t)resid) & 15) == 0) {
    const float* base = resid + j;
    int64_t r = r0;
    // whole groups: DIST_UNR unconditional loads issued before the first use (a per-load
    // condition here becomes a branch with its own wait, one load in flight at a time)
    for (; r + DIST_UNR <= r1; r += DIST_UNR) {
      float4 v[DIST_UNR];
#pragma unroll
      for (int u = 0; u < DIST_UNR; ++u)
        v[u] = *reinterpret_cast<const float4*>(base + (r + u) * ldr);
#pragma unroll
      for (int u = 0; u < DIST_UNR; ++u) {
        acc[0] = fma((double)v[u].x, (double)v[u].x, acc[0]);
        acc[1] = fma((double)v[u].y, (double)v[u].y, acc[1]);
        acc[2] = fma((double)v[u].z, (double)v[u].z, acc[2]);
        acc[3] = fma((double)v[u].w, (double)v[u].w, acc[3]);
      }
    }
    for (; r < r1; ++r) {
      const float4 v = *reinterpret_cast<const float4*>(base + r * ldr);
      acc[0] = fma((double)v.x, (double)v.x, acc[0]);
      acc[1] = fma((double)v.y, (double)v.y, acc[1]);
      acc[2] = fma((double)v.z, (double)v.z, acc[2]);
      acc[3] = fma((double)v.w, (double)v.w, acc[3]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j + e < n_in) {
#pragma unroll 8
        for (int64_t r = r0; r < r1; ++r) {
          const double v = (double)resid[r * ldr + j + e];
          acc[e] = fma(v, v, acc[e]);
        }
      }
    }
  }
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (j + e < n_in) {
      const double d = U[(j + e) * ldu + j + e];
      s = fma(acc[e], d * d, s);
    }
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void k_sum_partials(const double* partial, int64_t n,
                                                      double* out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// W_hat_ij = Delta_ij q_ij with Delta_ij = c / (U_jj rs_i) (rs_i = 1 without class scales; the
// SoftWater page, §2 "Aproximação Tratável", divides row i's grid by sqrt(lambda_i)), written as
// float or bf16 (round to nearest
// even).
template <bool BF16>
__global__ void k_dequant(const int32_t* __restrict__ codes, int64_t n_out, int64_t n_in,
                          int64_t ldq, const double* __restrict__ invd, double c, void* W_hat,
                          int64_t ldh, const double* __restrict__ rs) {
  const int64_t total = n_out * n_in;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / n_in, j = e % n_in;
    const double step = rs ? (c * invd[j]) / rs[r] : c * invd[j];
    const float v = (float)(step * (double)codes[r * ldq + j]);
    if (BF16) {
      uint32_t u = __float_as_uint(v);
      u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      ((uint16_t*)W_hat)[r * ldh + j] = (uint16_t)u;
    } else {
      ((float*)W_hat)[r * ldh + j] = v;
    }
  }
}

}  // namespace

int launch_dist_resid(const float* resid, int64_t n_out, int64_t n_in, int64_t ldr,
                      const double* U, int64_t ldu, double* partial, int nblk, hipStream_t st) {
  const unsigned gx = (unsigned)((n_in + DIST_COLS - 1) / DIST_COLS);
  const unsigned gy = (unsigned)((n_out + DIST_ROWS - 1) / DIST_ROWS);
  if ((int64_t)gx * gy > nblk) {
    set_error("internal: distortion partials %u x %u > %d", gx, gy, nblk);
    return WSIC_E_WORKSPACE;
  }
  WSIC_LAUNCH("dist_resid", 4.0 * (double)n_out * n_in, st, k_dist_resid, dim3(gx, gy), dim3(256),
              0, resid, n_out, n_in, ldr, U, ldu, partial);
  return WSIC_OK;
}

int launch_sum_partials(const double* partial, int64_t n, double* out, hipStream_t st) {
  WSIC_LAUNCH("sum_partials", 8.0 * n, st, k_sum_partials, dim3(1), dim3(256), 0, partial, n, out);
  return WSIC_OK;
}

int launch_dequant(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                   const double* invd, double c, void* W_hat, int w_hat_dtype, int64_t ldh,
                   hipStream_t st, const double* rs) {
  const int64_t total = n_out * n_in;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const double work = (double)total * (4.0 + (w_hat_dtype == WSIC_BF16 ? 2.0 : 4.0));
  if (w_hat_dtype == WSIC_BF16)
    WSIC_LAUNCH("dequant", work, st, k_dequant<true>, dim3((unsigned)blocks), dim3(256), 0, codes,
                n_out, n_in, ldq, invd, c, W_hat, ldh, rs);
  else
    WSIC_LAUNCH("dequant", work, st, k_dequant<false>, dim3((unsigned)blocks), dim3(256), 0, codes,
                n_out, n_in, ldq, invd, c, W_hat, ldh, rs);
  return WSIC_OK;
}

}  // namespace wsic
