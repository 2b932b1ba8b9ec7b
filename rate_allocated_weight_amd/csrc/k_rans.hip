// Entropy coder for the integer codes (WaterSIC page, §2 item 3: the codes are not clipped to a
// fixed range but compressed by an entropy coder, so the layer's rate is what the coder writes).
// Range-variant ANS with a static table from the pooled code histogram:
//   * 32-bit states in [2^16, 2^32), 16-bit renormalization, frequencies scaled to 2^14;
//   * the codes within +-2047 form the alphabet [lo, lo + nsym - 2], plus one escape symbol whose
//     code is stored raw (int32) in a side array;
//   * a group of 64 streams (one wave) holds a block of 64 L consecutive codes, lane l taking every
//     64th one, so that the decoder's loads of codes and stores of values are contiguous across the
//     wave at every step; the group's 16-bit words are stored in the order the decoder consumes
//     them (by step, then by lane among the lanes that read one), found with a wave ballot and a
//     prefix popcount, so the decoder's word loads are contiguous too.
//
//   k_rans_esc_count  escapes per group (for the escape offsets, scanned before encoding)
//   k_rans_encode     symbols in reverse order per lane; words written backwards into a per-group
//                     area, escapes straight into the container
//   k_scan_u32        exclusive prefix sums (one workgroup): word and escape offsets
//   k_rans_compact    each group's words into the container's payload
//   k_rans_decode     one wave per group, a 2^14-entry slot -> symbol table in LDS; writes int32
//                     codes, or dequantized weights c q / U_jj (float or bf16)
#include "common.h"

namespace wsic {
namespace {

constexpr int RPROB = 14, RM = 1 << RPROB, RLANES = 64, RWIN = 2047;
constexpr uint32_t RLOW = 1u << 16;

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

__global__ __launch_bounds__(256) void k_rans_esc_count(const int32_t* __restrict__ q, int64_t N,
                                                        int L, int64_t G,
                                                        uint32_t* __restrict__ cnt) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  uint32_t c = 0;
  for (int k = 0; k < L; ++k) {
    const int64_t p = (g * L + k) * RLANES + lane;
    if (p < N) {
      const int v = q[p];
      c += (v < -RWIN || v > RWIN) ? 1u : 0u;
    }
  }
  for (int d = 1; d < 64; d <<= 1) c += __shfl_xor(c, d, 64);
  if (lane == 0) cnt[g] = c;
}

__global__ __launch_bounds__(256) void k_rans_encode(const int32_t* __restrict__ q, int64_t N, int L,
                                                     int64_t G, int lo, int nsym,
                                                     const uint16_t* __restrict__ freq,
                                                     const uint32_t* __restrict__ eofs,
                                                     int32_t* __restrict__ esc_out,
                                                     uint16_t* __restrict__ temp,
                                                     uint32_t* __restrict__ gwords,
                                                     uint32_t* __restrict__ states) {
  __shared__ uint16_t sf[4096 + 8], sc[4096 + 8];
  for (int s = threadIdx.x; s < nsym; s += 256) sf[s] = freq[s];
  __syncthreads();
  if (threadIdx.x == 0) {  // cumulative frequencies (nsym <= 4096)
    uint32_t c = 0;
    for (int s = 0; s < nsym; ++s) {
      sc[s] = (uint16_t)c;
      c += sf[s];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  const int esc = nsym - 1;
  uint16_t* tw = temp + g * (int64_t)RLANES * L;
  int64_t tail = (int64_t)RLANES * L;
  const uint32_t e0 = eofs[g], etot = eofs[g + 1] - e0;
  uint32_t eafter = 0;
  uint32_t x = RLOW;
  const uint64_t below = lanes_below(lane);
  for (int k = L - 1; k >= 0; --k) {
    const int64_t p = (g * L + k) * RLANES + lane;
    const bool active = p < N;
    const int v = active ? q[p] : 0;
    const bool inw = v >= -RWIN && v <= RWIN;
    const int s = inw ? v - lo : esc;
    const uint64_t em = __ballot(active && !inw);
    const uint32_t ne = (uint32_t)__popcll(em);
    if (active && !inw) esc_out[e0 + etot - eafter - ne + (uint32_t)__popcll(em & below)] = v;
    eafter += ne;
    const uint32_t f = active ? sf[s] : 1u, c = active ? sc[s] : 0u;
    const bool emit = active && (uint64_t)x >= ((uint64_t)f << 18);  // f = 2^14: never
    const uint64_t wm = __ballot(emit);
    const int nw = __popcll(wm);
    if (emit) {
      tw[tail - nw + __popcll(wm & below)] = (uint16_t)(x & 0xffffu);
      x >>= 16;
    }
    tail -= nw;
    if (active) x = ((x / f) << RPROB) + (x % f) + c;
  }
  states[g * RLANES + lane] = x;
  if (lane == 0) gwords[g] = (uint32_t)((int64_t)RLANES * L - tail);
}

// out[0] = 0, out[i + 1] = in[0] + ... + in[i] (i < n); one workgroup of 1024 threads
__global__ __launch_bounds__(1024) void k_scan_u32(const uint32_t* __restrict__ in, int64_t n,
                                                   uint32_t* __restrict__ out) {
  __shared__ uint32_t pre[1024];
  __shared__ uint32_t base;
  const int t = threadIdx.x;
  if (t == 0) {
    base = 0;
    out[0] = 0;
  }
  __syncthreads();
  for (int64_t i0 = 0; i0 < n; i0 += 1024) {
    const int64_t i = i0 + t;
    pre[t] = i < n ? in[i] : 0u;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const uint32_t v = t >= d ? pre[t - d] : 0u;
      __syncthreads();
      pre[t] += v;
      __syncthreads();
    }
    if (i < n) out[i + 1] = base + pre[t];
    __syncthreads();
    if (t == 1023) base += pre[1023];
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_rans_compact(const uint16_t* __restrict__ temp, int L,
                                                      const uint32_t* __restrict__ gwords,
                                                      const uint32_t* __restrict__ gofs,
                                                      uint16_t* __restrict__ payload) {
  const int64_t g = blockIdx.x;
  const int64_t cap = (int64_t)RLANES * L;
  const uint32_t n = gwords[g];
  const uint16_t* src = temp + g * cap + (cap - n);
  uint16_t* dst = payload + gofs[g];
  for (uint32_t i = threadIdx.x; i < n; i += 256) dst[i] = src[i];
}

template <int MODE>  // 0: int32 codes; 1: float weights; 2: bf16 weights
__global__ __launch_bounds__(256) void k_rans_decode(const uint16_t* __restrict__ freq, int nsym, int lo,
                                                     int64_t N, int L, int64_t G,
                                                     const uint32_t* __restrict__ gofs,
                                                     const uint32_t* __restrict__ eofs,
                                                     const uint32_t* __restrict__ states,
                                                     const int32_t* __restrict__ escapes,
                                                     uint32_t n_esc,
                                                     const uint16_t* __restrict__ payload,
                                                     uint32_t n_words,
                                                     void* __restrict__ out, int64_t n_in,
                                                     const double* __restrict__ invd, double cscale,
                                                     int* __restrict__ flags) {
  __shared__ uint16_t lut[RM];
  __shared__ uint16_t sf[4096 + 8], sc[4096 + 8];
  for (int s = threadIdx.x; s < nsym; s += 256) sf[s] = freq[s];
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t c = 0;
    for (int s = 0; s < nsym; ++s) {
      sc[s] = (uint16_t)c;
      c += sf[s];
    }
  }
  __syncthreads();
  for (int slot = threadIdx.x; slot < RM; slot += 256) {  // largest s with cum[s] <= slot, f > 0
    int a = 0, b = nsym - 1;
    while (a < b) {
      const int m = (a + b + 1) >> 1;
      if (sc[m] <= slot) a = m;
      else b = m - 1;
    }
    while (a > 0 && sf[a] == 0) --a;  // zero-frequency symbols share their successor's cumulative
    lut[slot] = (uint16_t)a;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  const int esc = nsym - 1;
  uint32_t x = states[g * RLANES + lane];
  uint32_t wp = gofs[g], ep = eofs[g];
  const uint64_t below = lanes_below(lane);
  int64_t col = MODE != 0 ? ((g * L) * RLANES + lane) % n_in : 0;
  for (int k = 0; k < L; ++k) {
    const int64_t p = (g * L + k) * RLANES + lane;
    const bool active = p < N;
    const uint32_t slot = x & (RM - 1);
    const int s = lut[slot];
    if (active) x = (uint32_t)sf[s] * (x >> RPROB) + slot - sc[s];
    const bool isesc = active && s == esc;
    const uint64_t em = __ballot(isesc);
    int v = lo + s;
    bool bad = false;  // reads past the escapes or the payload: a corrupt container
    if (isesc) {
      const uint32_t i = ep + (uint32_t)__popcll(em & below);
      bad |= i >= n_esc;
      v = i < n_esc ? escapes[i] : 0;
    }
    ep += (uint32_t)__popcll(em);
    const bool need = active && x < RLOW;
    const uint64_t wm = __ballot(need);
    if (need) {
      const uint32_t i = wp + (uint32_t)__popcll(wm & below);
      bad |= i >= n_words;
      x = (x << 16) | (i < n_words ? payload[i] : 0u);
    }
    wp += (uint32_t)__popcll(wm);
    if (bad) atomicOr(flags, FLAG_RANGE);
    if (active) {
      if (MODE == 0) {
        ((int32_t*)out)[p] = v;
      } else {
        const float w = (float)((cscale * invd[col]) * (double)v);
        if (MODE == 1) {
          ((float*)out)[p] = w;
        } else {
          uint32_t u = __float_as_uint(w);
          u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
          ((uint16_t*)out)[p] = (uint16_t)u;
        }
      }
    }
    if (MODE != 0) {  // the column of the next step's weight
      col += RLANES;
      while (col >= n_in) col -= n_in;
    }
  }
  if (x != RLOW) atomicOr(flags, FLAG_RANGE);  // every stream ends in the encoder's start state
}

}  // namespace

int launch_rans_esc_count(const int32_t* q, int64_t N, int L, int64_t G, uint32_t* cnt, hipStream_t st) {
  WSIC_LAUNCH("rans_esc", 4.0 * (double)N, st, k_rans_esc_count, dim3((unsigned)((G + 3) / 4)), dim3(256),
              0, q, N, L, G, cnt);
  return WSIC_OK;
}

int launch_scan_u32(const uint32_t* in, int64_t n, uint32_t* out, hipStream_t st) {
  WSIC_LAUNCH("scan", 8.0 * (double)n, st, k_scan_u32, dim3(1), dim3(1024), 0, in, n, out);
  return WSIC_OK;
}

int launch_rans_encode(const int32_t* q, int64_t N, int L, int64_t G, int lo, int nsym,
                       const uint16_t* freq, const uint32_t* eofs, int32_t* esc_out, uint16_t* temp,
                       uint32_t* gwords, uint32_t* states, hipStream_t st) {
  if (nsym > 4096) return WSIC_E_INVAL;
  WSIC_LAUNCH("rans_encode", 4.0 * (double)N, st, k_rans_encode, dim3((unsigned)((G + 3) / 4)),
              dim3(256), 0, q, N, L, G, lo, nsym, freq, eofs, esc_out, temp, gwords, states);
  return WSIC_OK;
}

int launch_rans_compact(const uint16_t* temp, int L, int64_t G, const uint32_t* gwords,
                        const uint32_t* gofs, uint16_t* payload, hipStream_t st) {
  WSIC_LAUNCH("rans_compact", 4.0 * (double)G * RLANES * L, st, k_rans_compact, dim3((unsigned)G),
              dim3(256), 0, temp, L, gwords, gofs, payload);
  return WSIC_OK;
}

int launch_rans_decode(int mode, const uint16_t* freq, int nsym, int lo, int64_t N, int L, int64_t G,
                       const uint32_t* gofs, const uint32_t* eofs, const uint32_t* states,
                       const int32_t* escapes, uint32_t n_esc, const uint16_t* payload,
                       uint32_t n_words, void* out, int64_t n_in, const double* invd, double c,
                       int* flags, hipStream_t st) {
  if (nsym > 4096) return WSIC_E_INVAL;
  const dim3 grid((unsigned)((G + 3) / 4));
  const double work = (double)N * (mode == 0 ? 4.0 : (mode == 1 ? 4.0 : 2.0));
  if (mode == 0)
    WSIC_LAUNCH("rans_decode", work, st, k_rans_decode<0>, grid, dim3(256), 0, freq, nsym, lo, N, L, G,
                gofs, eofs, states, escapes, n_esc, payload, n_words, out, n_in, invd, c, flags);
  else if (mode == 1)
    WSIC_LAUNCH("rans_decode", work, st, k_rans_decode<1>, grid, dim3(256), 0, freq, nsym, lo, N, L, G,
                gofs, eofs, states, escapes, n_esc, payload, n_words, out, n_in, invd, c, flags);
  else
    WSIC_LAUNCH("rans_decode", work, st, k_rans_decode<2>, grid, dim3(256), 0, freq, nsym, lo, N, L, G,
                gofs, eofs, states, escapes, n_esc, payload, n_words, out, n_in, invd, c, flags);
  return WSIC_OK;
}

}  // namespace wsic
