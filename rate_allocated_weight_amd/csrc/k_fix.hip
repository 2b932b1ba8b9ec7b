// Practical corrections of the WaterSIC page, §2 item 4:
//   * "Correzione LMMSE": one factor per output row rescales the quantized row,
//     gamma_k = (w_k Sigma w_hat_k^T) / (w_hat_k Sigma w_hat_k^T). With y = U w^T (Y = W U^T) and
//     the SIC identity (U (w - w_hat)^T)_j = U_jj r_j, U w_hat^T = y - diag(U) r, so the three
//     inner products stream Y and the residuals once (k_lmmse_rows).
//   * "Cancellazione delle Feature Morte": input columns of near-zero variance are taken out of the
//     problem: k_live_scan lists the columns with Sigma_ii > tau max_j Sigma_jj (one workgroup,
//     ascending order) and each column's position in that list (-1: dead), k_gather_* build the
//     live layer and covariance, k_scatter_codes writes every column of the full code matrix once
//     (the live code, or 0 for a dead column).
#include "common.h"

namespace wsic {
namespace {

// one 256-thread workgroup per row; fp64 sums over the row, deterministic tree reduction
__global__ __launch_bounds__(256) void k_lmmse_rows(const double* __restrict__ Y, int64_t ldy,
                                                    const float* __restrict__ R, int64_t ldr,
                                                    const double* __restrict__ U, int64_t ldu,
                                                    int64_t n_in, double* __restrict__ gamma,
                                                    double* __restrict__ dbefore,
                                                    double* __restrict__ dafter) {
  __shared__ double ra[256], rb[256], rw[256];
  const int64_t row = blockIdx.x;
  double a = 0.0, b = 0.0, w = 0.0;
  for (int64_t j = threadIdx.x; j < n_in; j += 256) {
    const double y = Y[row * ldy + j];
    const double h = y - U[j * ldu + j] * (double)R[row * ldr + j];  // (U w_hat^T)_j
    a = fma(y, h, a);
    b = fma(h, h, b);
    w = fma(y, y, w);
  }
  ra[threadIdx.x] = a;
  rb[threadIdx.x] = b;
  rw[threadIdx.x] = w;
  __syncthreads();
  for (int d = 128; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) {
      ra[threadIdx.x] += ra[threadIdx.x + d];
      rb[threadIdx.x] += rb[threadIdx.x + d];
      rw[threadIdx.x] += rw[threadIdx.x + d];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double A = ra[0], B = rb[0], WW = rw[0];
    const double before = WW - 2.0 * A + B;
    const bool zero = !(B > 0.0);
    gamma[row] = zero ? 1.0 : A / B;
    dbefore[row] = before;
    dafter[row] = zero ? before : WW - A * A / B;
  }
}

// live columns in ascending order; n_live in live_count[0]; one workgroup of 1024 threads
__global__ __launch_bounds__(1024) void k_live_scan(const double* __restrict__ S, int64_t n,
                                                    int64_t lds, double tau,
                                                    int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ pos,
                                                    long long* __restrict__ live_count,
                                                    int* __restrict__ flags) {
  __shared__ double mx[1024];
  __shared__ int pre[1024];
  __shared__ long long base;
  const int t = threadIdx.x;
  double m = 0.0;
  for (int64_t i = t; i < n; i += 1024) {
    const double d = S[i * lds + i];
    if (!isfinite(d)) atomicOr(flags, FLAG_NONFINITE);
    m = fmax(m, d);
  }
  mx[t] = m;
  __syncthreads();
  for (int d = 512; d >= 1; d >>= 1) {
    if (t < d) mx[t] = fmax(mx[t], mx[t + d]);
    __syncthreads();
  }
  const double thr = tau * mx[0];
  if (t == 0) base = 0;
  __syncthreads();
  for (int64_t i0 = 0; i0 < n; i0 += 1024) {
    const int64_t i = i0 + t;
    const int live = (i < n) && (S[i * lds + i] > thr) ? 1 : 0;
    pre[t] = live;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan (Hillis-Steele)
      const int v = t >= d ? pre[t - d] : 0;
      __syncthreads();
      pre[t] += v;
      __syncthreads();
    }
    if (live) idx[base + pre[t] - 1] = (int32_t)i;
    if (i < n) pos[i] = live ? (int32_t)(base + pre[t] - 1) : -1;
    __syncthreads();
    if (t == 1023) base += pre[1023];
    __syncthreads();
  }
  if (t == 0) live_count[0] = base;
}

template <typename T>
__global__ void k_gather_w(const T* __restrict__ W, int64_t n_out, int64_t ldw,
                           const int32_t* __restrict__ idx, int64_t n_live, T* __restrict__ Wl,
                           int64_t ldl) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (j < n_live) Wl[r * ldl + j] = W[r * ldw + idx[j]];
}

__global__ void k_gather_sigma(const double* __restrict__ S, int64_t lds,
                               const int32_t* __restrict__ idx, int64_t n_live,
                               double* __restrict__ Sl, int64_t ldsl) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = blockIdx.y;
  if (j < n_live) Sl[i * ldsl + j] = S[(int64_t)idx[i] * lds + idx[j]];
}

__global__ void k_scatter_codes(const int32_t* __restrict__ ql, int64_t ldql,
                                const int32_t* __restrict__ pos, int64_t n_in,
                                int32_t* __restrict__ q, int64_t ldq) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (j < n_in) {
    const int p = pos[j];
    q[r * ldq + j] = p >= 0 ? ql[r * ldql + p] : 0;
  }
}

// Rows of the rate controller's probe layer: row g * S + i is row r_i = floor((2 i + 1) n_out /
// (2 S)) of Y times fac.v[g] (the probe's grid scale c_g enters as Y / c_g = (Y c / c_g) / c).
__global__ void k_probe_rows(const double* __restrict__ Y, int64_t ldy, int64_t n_out, int64_t n_in,
                             int S, ProbeFactors fac, double* __restrict__ Yp, int64_t ldp) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int v = blockIdx.y, g = v / S, i = v - g * S;
  const int64_t r = ((2 * (int64_t)i + 1) * n_out) / (2 * (int64_t)S);
  if (j < n_in) Yp[(int64_t)v * ldp + j] = Y[r * ldy + j] * fac.v[g];
}

}  // namespace

int launch_lmmse_rows(const double* Y, int64_t ldy, const float* R, int64_t ldr, const double* U,
                      int64_t ldu, int64_t n_out, int64_t n_in, double* gamma, double* dbefore,
                      double* dafter, hipStream_t st) {
  if (n_out > 0x7fffffff) return WSIC_E_INVAL;
  WSIC_LAUNCH("lmmse_rows", 12.0 * (double)n_out * n_in, st, k_lmmse_rows, dim3((unsigned)n_out),
              dim3(256), 0, Y, ldy, R, ldr, U, ldu, n_in, gamma, dbefore, dafter);
  return WSIC_OK;
}

int launch_live_scan(const double* S, int64_t n, int64_t lds, double tau, int32_t* idx,
                     int32_t* pos, long long* live_count, int* flags, hipStream_t st) {
  WSIC_LAUNCH("live_scan", 16.0 * n, st, k_live_scan, dim3(1), dim3(1024), 0, S, n, lds, tau, idx,
              pos, live_count, flags);
  return WSIC_OK;
}

int launch_gather_features(const void* W, int dtype, int64_t n_out, int64_t ldw, const double* S,
                           int64_t lds, const int32_t* idx, int64_t n_live, void* Wl, int64_t ldwl,
                           double* Sl, int64_t ldsl, hipStream_t st) {
  const unsigned gx = (unsigned)((n_live + 255) / 256);
  for (int64_t r0 = 0; r0 < n_out; r0 += 65535) {
    const int64_t nr = n_out - r0 < 65535 ? n_out - r0 : 65535;
    if (dtype == WSIC_BF16)
      WSIC_LAUNCH("gather", 4.0 * (double)nr * n_live, st, k_gather_w<uint16_t>, dim3(gx, (unsigned)nr),
                  dim3(256), 0, (const uint16_t*)W + r0 * ldw, nr, ldw, idx, n_live,
                  (uint16_t*)Wl + r0 * ldwl, ldwl);
    else
      WSIC_LAUNCH("gather", 8.0 * (double)nr * n_live, st, k_gather_w<float>, dim3(gx, (unsigned)nr),
                  dim3(256), 0, (const float*)W + r0 * ldw, nr, ldw, idx, n_live,
                  (float*)Wl + r0 * ldwl, ldwl);
  }
  if (S) {
    if (n_live > 65535) return WSIC_E_INVAL;
    WSIC_LAUNCH("gather", 16.0 * (double)n_live * n_live, st, k_gather_sigma,
                dim3(gx, (unsigned)n_live), dim3(256), 0, S, lds, idx, n_live, Sl, ldsl);
  }
  return WSIC_OK;
}

int launch_scatter_codes(const int32_t* ql, int64_t ldql, const int32_t* pos, int64_t n_in,
                         int64_t n_out, int32_t* q, int64_t ldq, hipStream_t st) {
  const unsigned gx = (unsigned)((n_in + 255) / 256);
  for (int64_t r0 = 0; r0 < n_out; r0 += 65535) {
    const int64_t nr = n_out - r0 < 65535 ? n_out - r0 : 65535;
    WSIC_LAUNCH("scatter", 12.0 * (double)nr * n_in, st, k_scatter_codes, dim3(gx, (unsigned)nr),
                dim3(256), 0, ql + r0 * ldql, ldql, pos, n_in, q + r0 * ldq, ldq);
  }
  return WSIC_OK;
}

int launch_probe_rows(const double* Y, int64_t ldy, int64_t n_out, int64_t n_in, int S, int K,
                      const ProbeFactors& fac, double* Yp, int64_t ldp, hipStream_t st) {
  if (S <= 0 || K <= 0 || K > PROBE_MAX || (int64_t)S * K > 65535 || S > n_out) return WSIC_E_INVAL;
  const unsigned gx = (unsigned)((n_in + 255) / 256);
  WSIC_LAUNCH("probe_rows", 16.0 * (double)S * K * n_in, st, k_probe_rows,
              dim3(gx, (unsigned)(S * K)), dim3(256), 0, Y, ldy, n_out, n_in, S, fac, Yp, ldp);
  return WSIC_OK;
}

}  // namespace wsic
