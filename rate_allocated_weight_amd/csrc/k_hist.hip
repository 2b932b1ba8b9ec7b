// Code histogram and empirical entropy (WaterSIC page, Sommario tecnico §2 item 3: the
// integer codes are unbounded and entropy coded, so the rate is the entropy of the code
// histogram).
//
// k_hist: each workgroup counts its share of the codes in an LDS window of +-255 bins (wider
// codes, rare below ~8 bits per weight, go straight to the global window of +-HIST_HALF);
// codes in [-7, 7] (the bulk at 1-4 bits per weight) are first tallied in per-thread
// registers and summed over the wave, to avoid LDS atomic contention on a handful of bins.
// Window counts are then added to a global u64 window; codes outside the window are appended to
// an overflow list that the host counts exactly.
// k_entropy_reduce: one workgroup forms sum_k n_k log2 n_k over the window in fp64.
#include "common.h"

namespace wsic {
namespace {

// Codes in [-7, 7] (the bulk at 1-4 bits per weight) are tallied per thread without a branch:
// each code adds 1 << 4 t (t = code + 7, clamped to 15) to a 64-bit word of sixteen 4-bit
// counters, so a code costs a handful of VALU operations. Nibble 15 collects every code outside
// the range (its carry leaves the word and is dropped); such codes are counted again, one by one,
// on the slow path. At most NIB_GROUP codes go into the nibbles before they are spread into
// byte counters (even and odd nibbles apart, four registers of four bytes), and a thread counts at
// most HIST_PER_THREAD codes, so neither a nibble nor a byte can overflow. The wave sums are
// formed in 16-bit halves (at most 64 x 255).
constexpr int REG_LO = -7, REG_HI = 7;
constexpr int HIST_PER_THREAD = 255;
constexpr int NIB_GROUP = 12;
// codes per thread the launch aims at (at most HIST_PER_THREAD), and threads per workgroup: at
// the attention layer's size one 512-thread workgroup per CU. More, smaller workgroups measured
// slower (each adds one global atomic per occupied bin at its end), fewer left CUs idle.
constexpr int HIST_TARGET = 128;
constexpr int HIST_THREADS = 512;
// LDS window of a workgroup (codes beyond it go to the global window with global atomics)
constexpr int LDS_HALF = 255, LDS_BINS = 2 * LDS_HALF + 1;

struct Tally {
  uint32_t n_lo = 0, n_hi = 0;                  // sixteen 4-bit counters
  uint32_t e_lo = 0, e_hi = 0, o_lo = 0, o_hi = 0;  // byte counters: even / odd nibbles
  __device__ __forceinline__ void add(int v) {
    const unsigned t = min((unsigned)(v - REG_LO), 15u);
    const unsigned long long inc = 1ull << (t << 2);
    n_lo += (uint32_t)inc;
    n_hi += (uint32_t)(inc >> 32);
  }
  __device__ __forceinline__ void flush() {
    e_lo += n_lo & 0x0f0f0f0fu;
    o_lo += (n_lo >> 4) & 0x0f0f0f0fu;
    e_hi += n_hi & 0x0f0f0f0fu;
    o_hi += (n_hi >> 4) & 0x0f0f0f0fu;
    n_lo = n_hi = 0u;
  }
  // codes that fell outside [REG_LO, REG_HI] so far (byte 3 of o_hi is nibble 15)
  __device__ __forceinline__ uint32_t outside() const { return o_hi >> 24; }
};

__global__ __launch_bounds__(HIST_THREADS) void k_hist(const int32_t* __restrict__ codes, int64_t n_out,
                                              int64_t n_in, int64_t ldq,
                                              unsigned long long* __restrict__ bins,
                                              int32_t* __restrict__ ovf,
                                              unsigned int* __restrict__ ovf_count) {
  __shared__ unsigned int lb[LDS_BINS];
  for (int b = threadIdx.x; b < LDS_BINS; b += blockDim.x) lb[b] = 0u;
  __syncthreads();

  Tally tl;
  // a code outside the register range: LDS window, else global window, else overflow list
  auto rare = [&](int v) {
    if (v >= REG_LO && v <= REG_HI) return;
    if (v >= -LDS_HALF && v <= LDS_HALF) {
      atomicAdd(&lb[v + LDS_HALF], 1u);
    } else if (v >= -HIST_HALF && v <= HIST_HALF) {
      atomicAdd(&bins[v + HIST_HALF], 1ull);
    } else {
      const unsigned int slot = atomicAdd(ovf_count, 1u);
      if (slot < OVF_CAP) ovf[slot] = v;
    }
  };
  auto one = [&](int v) {
    tl.add(v);
    tl.flush();
    rare(v);
  };
  const int64_t total = n_out * n_in;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (ldq == n_in && (((uintptr_t)codes) & 15) == 0) {
    // dense: 16-byte loads, UNR of them per batch; the next batch's loads are issued before the
    // current batch is counted (two register buffers), so a wave always has loads in flight
    constexpr int UNR = 8;
    const int4* c4 = reinterpret_cast<const int4*>(codes);
    const int64_t n4 = total / 4;
    const int64_t S = stride * UNR;
    auto full = [&](int64_t x) { return x + (UNR - 1) * stride < n4; };
    auto load = [&](int4* v, int64_t x) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) v[u] = c4[x + u * stride];
    };
    auto batch = [&](const int4* v) {
      const uint32_t before = tl.outside();
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        tl.add(v[u].x);
        tl.add(v[u].y);
        tl.add(v[u].z);
        tl.add(v[u].w);
        if ((u + 1) % (NIB_GROUP / 4) == 0 || u == UNR - 1) tl.flush();
      }
      // slow path, taken by the whole wave when any of its lanes saw a code outside the range
      if (__ballot(tl.outside() != before) != 0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          rare(v[u].x);
          rare(v[u].y);
          rare(v[u].z);
          rare(v[u].w);
        }
      }
    };
    int64_t e = gid;
    int4 a[UNR], b[UNR];
    if (full(e)) load(a, e);
    while (full(e)) {
      if (full(e + S)) load(b, e + S);
      batch(a);
      e += S;
      if (!full(e)) break;
      if (full(e + S)) load(a, e + S);
      batch(b);
      e += S;
    }
    for (; e < n4; e += stride) {
      const int4 v = c4[e];
      one(v.x);
      one(v.y);
      one(v.z);
      one(v.w);
    }
    for (int64_t k = n4 * 4 + gid; k < total; k += stride) one(codes[k]);
  } else {
    for (int64_t k = gid; k < total; k += stride) one(codes[(k / n_in) * ldq + (k % n_in)]);
  }
  // byte counters -> 16-bit halves (bytes 0 and 2, then 1 and 3), summed over the wave, one LDS
  // atomic per wave and bin. Byte b of e_lo holds t = 2b, of e_hi 8 + 2b, of o_lo 2b + 1, of
  // o_hi 9 + 2b (t = 15 is the out-of-range nibble and is not a bin).
  const int lane = threadIdx.x & 63;
  const uint32_t regs[4] = {tl.e_lo, tl.e_hi, tl.o_lo, tl.o_hi};
  const int t0[4] = {0, 8, 1, 9};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      unsigned int v = (regs[k] >> (8 * odd)) & 0x00ff00ffu;
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == 0) {
        const int ta = t0[k] + 2 * odd;      // byte odd
        const int tb = t0[k] + 2 * (odd + 2);  // byte odd + 2
        if (v & 0xffffu) atomicAdd(&lb[ta + REG_LO + LDS_HALF], v & 0xffffu);
        if ((v >> 16) && tb < 15) atomicAdd(&lb[tb + REG_LO + LDS_HALF], v >> 16);
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
  int64_t blocks = (total + HIST_THREADS * HIST_TARGET - 1) / (HIST_THREADS * HIST_TARGET);
  const int64_t per = HIST_PER_THREAD - 7;
  const int64_t need = (total + (int64_t)HIST_THREADS * per - 1) / ((int64_t)HIST_THREADS * per);
  if (blocks > 2048) blocks = 2048;
  if (blocks < need) blocks = need;
  if (blocks < 1) blocks = 1;
  WSIC_LAUNCH("hist", 4.0 * (double)total, st, k_hist, dim3((unsigned)blocks), dim3(HIST_THREADS), 0,
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
