// Code histogram and empirical entropy (WaterSIC page, Sommario tecnico §2 item 3: the
// integer codes are unbounded and entropy coded, so the rate is the entropy of the code
// histogram).
//
// k_hist: each workgroup counts its share of the codes in an LDS window of +-255 bins (wider
// codes, rare below ~8 bits per weight, go straight to the global window of +-HIST_HALF);
// codes in [-7, 8] (the bulk at 1-4 bits per weight) are first tallied in per-thread
// registers and summed over the wave, to avoid LDS atomic contention on a handful of bins.
// Window counts are then added to a global u64 window; codes outside the window are appended to
// an overflow list that the host counts exactly.
// k_entropy_reduce: one workgroup forms sum_k n_k log2 n_k over the window in fp64.
#include "common.h"

namespace wsic {
namespace {

// codes in [-7, 8] are tallied per thread as 8-bit counters, four to a register; a thread
// counts at most HIST_PER_THREAD codes, so a counter cannot overflow, and the wave sums are
// formed in 16-bit halves (at most 64 x 255)
constexpr int REG_LO = -7, REG_N = 16;
constexpr int HIST_PER_THREAD = 255;
// LDS window of a workgroup (codes beyond it go to the global window with global atomics)
constexpr int LDS_HALF = 255, LDS_BINS = 2 * LDS_HALF + 1;

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ codes, int64_t n_out,
                                              int64_t n_in, int64_t ldq,
                                              unsigned long long* __restrict__ bins,
                                              int32_t* __restrict__ ovf,
                                              unsigned int* __restrict__ ovf_count) {
  __shared__ unsigned int lb[LDS_BINS];
  for (int b = threadIdx.x; b < LDS_BINS; b += blockDim.x) lb[b] = 0u;
  __syncthreads();

  unsigned int reg[REG_N / 4];
#pragma unroll
  for (int k = 0; k < REG_N / 4; ++k) reg[k] = 0u;

  auto count = [&](int v) {
    const int t = v - REG_LO;
    if ((unsigned)t < (unsigned)REG_N) {
      const unsigned int inc = 1u << (8 * (t & 3));
#pragma unroll
      for (int k = 0; k < REG_N / 4; ++k) reg[k] += ((t >> 2) == k) ? inc : 0u;
    } else if (v >= -LDS_HALF && v <= LDS_HALF) {
      atomicAdd(&lb[v + LDS_HALF], 1u);
    } else if (v >= -HIST_HALF && v <= HIST_HALF) {
      atomicAdd(&bins[v + HIST_HALF], 1ull);
    } else {
      const unsigned int slot = atomicAdd(ovf_count, 1u);
      if (slot < OVF_CAP) ovf[slot] = v;
    }
  };
  const int64_t total = n_out * n_in;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (ldq == n_in && (((uintptr_t)codes) & 15) == 0) {
    // dense: 16-byte loads, UNR of them in flight per thread
    constexpr int UNR = 8;
    const int4* c4 = reinterpret_cast<const int4*>(codes);
    const int64_t n4 = total / 4;
    for (int64_t e = gid; e < n4; e += stride * UNR) {
      int4 v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) v[u] = (e + u * stride < n4) ? c4[e + u * stride] : make_int4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (e + u * stride < n4) {
          count(v[u].x);
          count(v[u].y);
          count(v[u].z);
          count(v[u].w);
        }
      }
    }
    for (int64_t e = n4 * 4 + gid; e < total; e += stride) count(codes[e]);
  } else {
    for (int64_t e = gid; e < total; e += stride) count(codes[(e / n_in) * ldq + (e % n_in)]);
  }
  // register tallies: widened to 16-bit halves (bins 4k, 4k+2 and 4k+1, 4k+3), summed over the
  // wave, one LDS atomic per wave and bin
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < REG_N / 4; ++k) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      unsigned int v = (reg[k] >> (8 * odd)) & 0x00ff00ffu;
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == 0) {
        const int b0 = 4 * k + odd + REG_LO + LDS_HALF;
        if (v & 0xffffu) atomicAdd(&lb[b0], v & 0xffffu);
        if (v >> 16) atomicAdd(&lb[b0 + 2], v >> 16);
      }
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < LDS_BINS; b += blockDim.x)
    if (lb[b]) atomicAdd(&bins[b - LDS_HALF + HIST_HALF], (unsigned long long)lb[b]);
}

__global__ __launch_bounds__(256) void k_entropy_reduce(const unsigned long long* bins,
                                                        const unsigned int* ovf_count,
                                                        const int* flags, EntropyResult* res) {
  __shared__ double sd[256];
  __shared__ unsigned long long sn[256];
  double s = 0.0;
  unsigned long long nsym = 0;
  for (int b = threadIdx.x; b < HIST_BINS; b += blockDim.x) {
    const unsigned long long n = bins[b];
    if (n) {
      s += (double)n * log2((double)n);
      ++nsym;
    }
  }
  sd[threadIdx.x] = s;
  sn[threadIdx.x] = nsym;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      sd[threadIdx.x] += sd[threadIdx.x + off];
      sn[threadIdx.x] += sn[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    res->sum_nlogn = sd[0];
    res->nsym = sn[0];
    res->ovf_count = *ovf_count;
    res->flags = flags ? flags[0] : 0;
    res->aux = flags ? flags[1] : 0;
    res->aux2 = flags ? flags[2] : 0;
  }
}

__global__ void k_fill_zero(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

int launch_hist(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                unsigned long long* bins, int32_t* ovf, unsigned int* ovf_count, hipStream_t st) {
  const int64_t total = n_out * n_in;
  // enough threads that none counts more than HIST_PER_THREAD codes (8-bit tallies): a thread
  // takes at most 4 ceil(total / (4 threads)) codes of the vector loop plus one of the tail, so
  // sizing for HIST_PER_THREAD - 7 per thread keeps it below the limit; about 128 codes per
  // thread otherwise, so the per-workgroup window clear and flush stay small
  int64_t blocks = (total + 256 * 128 - 1) / (256 * 128);
  const int64_t per = HIST_PER_THREAD - 7;
  const int64_t need = (total + 256LL * per - 1) / (256LL * per);
  if (blocks > 2048) blocks = 2048;
  if (blocks < need) blocks = need;
  if (blocks < 1) blocks = 1;
  WSIC_LAUNCH("hist", 4.0 * (double)total, st, k_hist, dim3((unsigned)blocks), dim3(256), 0,
              codes, n_out, n_in, ldq, bins, ovf, ovf_count);
  return WSIC_OK;
}

int launch_entropy_reduce(const unsigned long long* bins, const unsigned int* ovf_count,
                          const int* flags, EntropyResult* res, hipStream_t st) {
  WSIC_LAUNCH("entropy", 8.0 * HIST_BINS, st, k_entropy_reduce, dim3(1), dim3(256), 0, bins,
              ovf_count, flags, res);
  return WSIC_OK;
}

// Zero-fill with a kernel (not hipMemsetAsync) so the call stays valid inside graph capture.
int launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return WSIC_OK;
  if (bytes % 4 != 0) {
    set_error("internal: fill of %zu bytes", bytes);
    return WSIC_E_INVAL;
  }
  const size_t words = bytes / 4;
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  WSIC_LAUNCH("fill_zero", (double)bytes, st, k_fill_zero, dim3((unsigned)blocks), dim3(256), 0,
              (uint32_t*)p, words);
  return WSIC_OK;
}

}  // namespace wsic
