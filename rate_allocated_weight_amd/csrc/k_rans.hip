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
//   k_rans_esc_count  escapes per group (for the escape offsets, scanned before encoding); one
//                     workgroup per group, 16-byte loads
//   k_rans_encode     symbols in reverse order per lane, the codes of the next 32 steps loading
//                     while 32 steps run; words written backwards into a per-group area, escapes
//                     straight into the container; xs / f through a per-symbol reciprocal in fp64
//                     with one exact correction
//   k_scan_u32        exclusive prefix sums (one workgroup): word and escape offsets
//   k_rans_compact    each group's words into the container's payload
//   k_rans_decode     eight groups (waves) per workgroup sharing two slot tables in LDS, built in
//                     parallel (frequency sums by a scan, each symbol marking its first slot, a
//                     prefix maximum spreading the marks): slot -> symbol, and slot -> (f, slot -
//                     cum) so that one LDS read gives the state update; the payload words reach the
//                     wave through a ring in LDS filled ahead of the decoder, so a step waits on LDS
//                     only; writes int32 codes, or dequantized weights c q / U_jj (float or bf16)
//                     with the column scales in LDS (n_in <= 4096) or loaded a block ahead
#include <type_traits>

#include "common.h"

namespace wsic {
namespace {

constexpr int RPROB = 14, RM = 1 << RPROB, RLANES = 64, RWIN = 2047;
constexpr uint32_t RLOW = 1u << 16;

// ballots and the count of the set lanes below this one, straight from the lane masks
__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t is_escape(int v) { return (v < -RWIN || v > RWIN) ? 1u : 0u; }

// Escapes per group: a group's L x 64 codes are contiguous, so one workgroup per group reads them
// with 16-byte loads (VEC: the codes are 16-byte aligned, which makes every group start so), eight
// loads in flight per thread, and sums the counts.
template <bool VEC>
__global__ __launch_bounds__(256) void k_rans_esc_count(const int32_t* __restrict__ q, int64_t N,
                                                        int L, int64_t G,
                                                        uint32_t* __restrict__ cnt) {
  __shared__ uint32_t part[4];
  const int64_t g = blockIdx.x;
  const int64_t e0 = g * (int64_t)L * RLANES;
  const int64_t e1 = e0 + (int64_t)L * RLANES < N ? e0 + (int64_t)L * RLANES : N;
  uint32_t c = 0;
  const int64_t n4 = VEC && e1 > e0 ? (e1 - e0) / 4 : 0;
  if (VEC) {
    const int4* q4 = reinterpret_cast<const int4*>(q + e0);
    for (int64_t i = threadIdx.x; i < n4; i += 256 * 8) {
      int4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t ii = i + u * 256;
        v[u] = q4[ii < n4 ? ii : n4 - 1];  // (clamped: counted only when in range)
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t m = (i + u * 256 < n4) ? 1u : 0u;
        c += m * (is_escape(v[u].x) + is_escape(v[u].y) + is_escape(v[u].z) + is_escape(v[u].w));
      }
    }
  }
  for (int64_t e = e0 + n4 * 4 + threadIdx.x; e < e1; e += 256) c += is_escape(q[e]);
  for (int d = 1; d < 64; d <<= 1) c += __shfl_xor(c, d, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) cnt[g] = (part[0] + part[1]) + (part[2] + part[3]);
}

// Exclusive prefix sums of the frequency table (nsym <= 4096) into sc, by a workgroup of NT threads
// (4096 / NT consecutive symbols each, then a scan of the thread sums); returns the table's total.
// Every thread of the workgroup calls it.
template <int NT>
__device__ uint32_t table_cum(const uint16_t* sf, uint16_t* sc, int nsym, uint32_t* wsum) {
  constexpr int PER = 4096 / NT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (t * PER + j < nsym) loc += sf[t * PER + j];
  uint32_t inc = loc;
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t c = inc - loc, total = 0;
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) c += wsum[i];
    total += wsum[i];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (t * PER + j < nsym) {
      sc[t * PER + j] = (uint16_t)c;
      c += sf[t * PER + j];
    }
  __syncthreads();
  return total;
}

constexpr int EB = 32;  // encoder: the codes of the next EB steps are loaded while EB steps run

__global__ __launch_bounds__(256) void k_rans_encode(const int32_t* __restrict__ q, int64_t N, int L,
                                                     int64_t G, int lo, int nsym,
                                                     const uint16_t* __restrict__ freq,
                                                     const uint32_t* __restrict__ eofs,
                                                     int32_t* __restrict__ esc_out,
                                                     uint16_t* __restrict__ temp,
                                                     uint32_t* __restrict__ gwords,
                                                     uint32_t* __restrict__ states) {
  __shared__ uint16_t sf[4096 + 8], sc[4096 + 8];
  __shared__ double srf[4096];  // 1 / f (0 for an absent symbol)
  __shared__ uint32_t wsum[4];
  for (int s = threadIdx.x; s < nsym; s += 256) {
    const uint16_t f = freq[s];
    sf[s] = f;
    srf[s] = f ? 1.0 / (double)f : 0.0;
  }
  __syncthreads();
  (void)table_cum<256>(sf, sc, nsym, wsum);
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  const int esc = nsym - 1;
  uint16_t* tw = temp + g * (int64_t)RLANES * L;
  int64_t tail = (int64_t)RLANES * L;
  const uint32_t e0 = eofs[g], etot = eofs[g + 1] - e0;
  uint32_t eafter = 0;
  uint32_t x = RLOW;
  const int64_t pbase = g * (int64_t)L * RLANES + lane;  // this lane's code at step 0
  // steps k < kact hold a code for this lane (all of them but in the last group's tail)
  const int kact = pbase < N ? (int)min((int64_t)L, (N - pbase + RLANES - 1) / RLANES) : 0;
  // block b holds steps k = L - 1 - EB b - j, j < EB (the symbols are encoded in reverse)
  auto load_block = [&](int b, int32_t(&dst)[EB]) {
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int k = L - 1 - EB * b - j;
      dst[j] = (k >= 0 && k < kact) ? q[pbase + (int64_t)k * RLANES] : 0;
    }
  };
  const int nblk = (L + EB - 1) / EB;
  int32_t nxt[EB];
  load_block(0, nxt);
  for (int b = 0; b < nblk; ++b) {
    int32_t cur[EB];
#pragma unroll
    for (int j = 0; j < EB; ++j) cur[j] = nxt[j];
    if (b + 1 < nblk) load_block(b + 1, nxt);
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int k = L - 1 - EB * b - j;
      if (k < 0) continue;  // (the last block's end; wave-uniform)
      const bool active = k < kact;
      const int v = cur[j];
      const bool inw = v >= -RWIN && v <= RWIN;
      const int s = !active ? 0 : (inw ? v - lo : esc);
      const uint64_t em = ballot(active && !inw);
      if (em) {  // (rare) escaped codes go raw, backwards from the end of the group's escapes
        const uint32_t ne = (uint32_t)__popcll(em);
        if (active && !inw) esc_out[e0 + etot - eafter - ne + count_below(em)] = v;
        eafter += ne;
      }
      const uint32_t f = sf[s], c = sc[s];
      const double rf = srf[s];
      const bool emit = active && (x >> 18) >= f;  // x >= f 2^18 (never for f = 2^14)
      const uint64_t wm = ballot(emit);
      const int nw = __popcll(wm);
      if (emit) tw[tail - nw + count_below(wm)] = (uint16_t)(x & 0xffffu);
      tail -= nw;
      const uint32_t xs = emit ? x >> 16 : x;
      // xs / f and xs % f: the product with the rounded 1/f truncates to the quotient or one less
      // (one more would need a quotient near 2^38; here it is below 2^18), so one step corrects it
      uint32_t qd = (uint32_t)((double)xs * rf);
      uint32_t r = xs - qd * f;
      const bool up = r >= f;
      qd += up ? 1u : 0u;
      r -= up ? f : 0u;
      const uint32_t xn = (qd << RPROB) + r + c;
      x = active ? xn : x;
    }
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

constexpr int DW = 8;            // decoder: groups (waves) per workgroup, sharing the slot tables
constexpr int RSEG = 512;        // payload words per ring segment (8 per lane; the shift by 9 below)
constexpr int RRING = 2 * RSEG;  // per wave: a ring of two segments in LDS
constexpr int DB = 16;           // decoder: the column scales of the next DB steps load during DB steps
constexpr int SL_COLS = 4096;    // decoder: columns whose scales fit in LDS beside the tables


// The decoder's output for code v as stored bits: the code (MODE 0), or the weight c v / U_jj
// (scale = c / U_jj) as float (MODE 1) or bf16, rounded to nearest even from the float (MODE 2).
template <int MODE>
__device__ __forceinline__ uint32_t output_bits(double scale, int v) {
  if (MODE == 0) return (uint32_t)v;
  const uint32_t u = __float_as_uint((float)(scale * (double)v));
  if (MODE == 1) return u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// MODE 0: int32 codes; 1: float weights; 2: bf16 weights. SL: the column scales sit in LDS
// (n_in <= 4096), else they are loaded a block of steps ahead into registers.
template <int MODE, bool SL>
__global__ __launch_bounds__(64 * DW) void k_rans_decode(const uint16_t* __restrict__ freq, int nsym,
                                                         int lo, int64_t N, int L, int64_t G,
                                                         const uint32_t* __restrict__ gofs,
                                                         const uint32_t* __restrict__ eofs,
                                                         const uint32_t* __restrict__ states,
                                                         const int32_t* __restrict__ escapes,
                                                         uint32_t n_esc,
                                                         const uint16_t* __restrict__ payload,
                                                         uint32_t n_words,
                                                         void* __restrict__ out, int64_t n_in,
                                                         const double* __restrict__ invd,
                                                         double cscale, int* __restrict__ flags) {
  constexpr int NT = 64 * DW;
  __shared__ __attribute__((aligned(16))) uint32_t lut[RM];   // f | (slot - cum) << 15
  __shared__ __attribute__((aligned(16))) uint16_t lsym[RM];  // the slot's symbol
  // the payload rings; before decoding they hold the frequencies and their sums (4096 each)
  __shared__ __attribute__((aligned(16))) uint16_t ring[DW * RRING];
  static_assert(DW * RRING >= 2 * 4096, "the table build borrows the rings");
  __shared__ uint32_t wsum[DW];
  __shared__ double ssc[SL ? SL_COLS : 1];  // c / U_jj per column
  uint16_t* sf = ring;
  uint16_t* sc = ring + 4096;
  const int t = threadIdx.x;
  for (int s = t; s < nsym; s += NT) sf[s] = freq[s];
  __syncthreads();
  if (table_cum<NT>(sf, sc, nsym, wsum) != (uint32_t)RM) {  // the same verdict in every thread
    if (t == 0) atomicOr(flags, FLAG_RANGE);
    return;
  }
  // slot -> symbol: each present symbol marks the first slot of its range, and a prefix maximum
  // carries the mark over the range (marks grow with the slot, as the sums do)
  for (int i = t; i < RM / 8; i += NT) reinterpret_cast<uint4*>(lsym)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  for (int s = t; s < nsym; s += NT)
    if (sf[s] != 0) lsym[sc[s]] = (uint16_t)s;
  __syncthreads();
  {
    constexpr int PER = RM / NT;  // consecutive slots per thread
    static_assert(PER % 8 == 0, "whole 16-byte pieces");
    const int lane = t & 63, w = t >> 6;
    uint16_t m[PER];
#pragma unroll
    for (int h = 0; h < PER / 8; ++h) {
      const uint4 v = reinterpret_cast<const uint4*>(lsym + t * PER)[h];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[8 * h + 2 * e] = (uint16_t)(u[e] & 0xffffu);
        m[8 * h + 2 * e + 1] = (uint16_t)(u[e] >> 16);
      }
    }
    uint32_t run = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) run = max(run, (uint32_t)m[i]);
    uint32_t inc = run;
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(inc, d, 64);
      if (lane >= d) inc = max(inc, o);
    }
    const uint32_t before = __shfl_up(inc, 1, 64);
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    run = lane > 0 ? before : 0u;
    for (int i = 0; i < w; ++i) run = max(run, wsum[i]);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      run = max(run, (uint32_t)m[i]);
      m[i] = (uint16_t)run;
    }
#pragma unroll
    for (int h = 0; h < PER / 8; ++h) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (uint32_t)m[8 * h + 2 * e] | ((uint32_t)m[8 * h + 2 * e + 1] << 16);
      reinterpret_cast<uint4*>(lsym + t * PER)[h] = make_uint4(u[0], u[1], u[2], u[3]);
    }
#pragma unroll
    for (int h = 0; h < PER / 4; ++h) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * h + e, slot = t * PER + i;
        u[e] = (uint32_t)sf[m[i]] | ((uint32_t)(slot - sc[m[i]]) << 15);
      }
      reinterpret_cast<uint4*>(lut + t * PER)[h] = make_uint4(u[0], u[1], u[2], u[3]);
    }
  }
  if (SL)
    for (int c = t; c < n_in; c += NT) ssc[c] = cscale * invd[c];
  __syncthreads();
  const int lane = t & 63;
  const int64_t g = (int64_t)blockIdx.x * DW + (t >> 6);
  if (g >= G) return;
  const int esc = nsym - 1;
  uint16_t* rg = ring + (t >> 6) * RRING;
  uint32_t x = states[g * RLANES + lane];
  uint32_t ep = eofs[g];
  // Payload words through a ring of two 512-word segments per wave. The group's words start at
  // A, and wr counts those consumed. Segment h holds the words [A + 512 h, A + 512 (h + 1)) (zero
  // past the payload) in slot h & 1; segments below `filled` have been written, the next two
  // wait in registers (P0 the even one, P1 the odd one). Eight steps read at most 512 words,
  // [A + wr, A + wr + 512): checked every eighth step, the segment of wr + 511 has grown by at
  // most one, so writing one segment when it reaches `filled` keeps the next eight steps' words
  // in the ring, and the segment it replaces (filled - 2) lies behind wr. The words wait in
  // registers for at least two refills (16 steps) before they are written.
  const uint32_t A = gofs[g];
  uint32_t wr = 0;
  // (one word per 32-bit register: packing two would wait for the loads at once)
  auto word = [&](uint64_t i) -> uint32_t { return i < n_words ? (uint32_t)payload[i] : 0u; };
  uint32_t P0[8], P1[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    rg[64 * h + lane] = (uint16_t)word((uint64_t)A + 64 * h + lane);
    rg[RSEG + 64 * h + lane] = (uint16_t)word((uint64_t)A + RSEG + 64 * h + lane);
    P0[h] = word((uint64_t)A + 2 * RSEG + 64 * h + lane);
    P1[h] = word((uint64_t)A + 3 * RSEG + 64 * h + lane);
  }
  uint32_t filled = 2;
  __builtin_amdgcn_wave_barrier();
  const int64_t pbase = g * (int64_t)L * RLANES + lane;  // this lane's output at step 0
  // steps k < kact write an output for this lane (all of them but in the last group's tail)
  const int kact = pbase < N ? (int)min((int64_t)L, (N - pbase + RLANES - 1) / RLANES) : 0;
  const int step_col = MODE != 0 ? (int)(RLANES % n_in) : 0;  // the column moves by 64 per step
  int col = MODE != 0 ? (int)(pbase % n_in) : 0;  // this step's column (SL) or the next one loaded
  auto next_col = [&]() {
    col += step_col;
    col -= col >= n_in ? (int)n_in : 0;
  };
  auto load_scales = [&](int kb, double(&dst)[DB]) {
#pragma unroll
    for (int j = 0; j < DB; ++j) {
      dst[j] = kb + j < kact ? cscale * invd[col] : 0.0;
      next_col();
    }
  };
  constexpr bool PREF = MODE != 0 && !SL;
  double snxt[DB];
  if (PREF) load_scales(0, snxt);
  const uint32_t ep0 = ep;
  const int nblk = (L + DB - 1) / DB;
  // FULL: every lane writes at every step (every group but the last); TAIL: the last, partial
  // block of steps (L not a multiple of DB)
  auto block = [&](auto full_tag, auto tail_tag, int b) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    double scur[DB];
    if (PREF) {
#pragma unroll
      for (int j = 0; j < DB; ++j) scur[j] = snxt[j];
      if (b + 1 < nblk) load_scales((b + 1) * DB, snxt);
    }
#pragma unroll
    for (int j = 0; j < DB; ++j) {
      const int k = b * DB + j;
      if (TAIL && k >= L) continue;  // (wave-uniform)
      if ((j & 7) == 0 && ((wr + (RSEG - 1)) >> 9) >= filled) {  // wave-uniform
        const uint64_t nb = (uint64_t)A + (uint64_t)(filled + 2) * RSEG;
        if (filled & 1u) {
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            rg[RSEG + 64 * h + lane] = (uint16_t)P1[h];
            P1[h] = word(nb + 64 * h + lane);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            rg[64 * h + lane] = (uint16_t)P0[h];
            P0[h] = word(nb + 64 * h + lane);
          }
        }
        ++filled;
        __builtin_amdgcn_wave_barrier();
      }
      const bool active = FULL || k < kact;
      const uint32_t slot = x & (RM - 1);
      const uint32_t e = lut[slot];
      const int s = lsym[slot];
      double scale = 0.0;
      if (MODE != 0) {
        if (SL) {
          scale = ssc[col];
          next_col();
        } else {
          scale = scur[j];
        }
      }
      // the state's chain first (update, renormalization word); the symbol's work after it
      const uint32_t xn = (e & 0x7fffu) * (x >> RPROB) + (e >> 15);
      x = active ? xn : x;
      const bool need = active && x < RLOW;
      const uint64_t wm = ballot(need);
      // (wr plus the needing lanes below, in the two mbcnt steps)
      const uint32_t w = rg[__builtin_amdgcn_mbcnt_hi((uint32_t)(wm >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)wm, wr)) &
                            (RRING - 1)];
      // the output of the table's symbol, formed while the word is read (an escaped lane's is
      // formed again below)
      int v = lo + s;
      uint32_t ov = output_bits<MODE>(scale, v);
      x = need ? ((x << 16) | w) : x;
      wr += (uint32_t)__popcll(wm);
      const bool isesc = active && s == esc;
      const uint64_t em = ballot(isesc);
      if (em) {  // (rare) the escaped codes; waited for here so that the store below never waits
        if (isesc) {
          const uint32_t i = ep + count_below(em);
          v = i < n_esc ? escapes[i] : 0;
          ov = output_bits<MODE>(scale, v);
        }
        asm volatile("" : "+v"(ov));
        ep += (uint32_t)__popcll(em);
      }
      if (active) {
        const int64_t p = pbase + (int64_t)k * RLANES;
        if (MODE == 0) ((int32_t*)out)[p] = (int32_t)ov;
        else if (MODE == 1) ((uint32_t*)out)[p] = ov;
        else ((uint16_t*)out)[p] = (uint16_t)ov;
      }
    }
  };
  auto run = [&](auto full_tag) {
    const int nwhole = L / DB;
    for (int b = 0; b < nwhole; ++b) block(full_tag, std::false_type{}, b);
    if (nwhole < nblk) block(full_tag, std::true_type{}, nwhole);
  };
  if ((g + 1) * (int64_t)L * RLANES <= N) run(std::true_type{});
  else run(std::false_type{});
  // A read past the payload or the escapes (a corrupt container) happened exactly when the group
  // consumed past their ends (the largest index read is the last one consumed); every stream ends
  // in the encoder's start state.
  const bool bad = (uint64_t)A + wr > (uint64_t)n_words ||
                   (uint64_t)ep0 + (uint32_t)(ep - ep0) > (uint64_t)n_esc;
  if (bad || x != RLOW) atomicOr(flags, FLAG_RANGE);
}

}  // namespace

int launch_rans_esc_count(const int32_t* q, int64_t N, int L, int64_t G, uint32_t* cnt, hipStream_t st) {
  if (G <= 0) return WSIC_OK;
  if (G > 0x7fffffff) {
    set_error("internal: %lld coder groups", (long long)G);
    return WSIC_E_INVAL;
  }
  if ((((uintptr_t)q) & 15) == 0)
    WSIC_LAUNCH("rans_esc", 4.0 * (double)N, st, k_rans_esc_count<true>, dim3((unsigned)G), dim3(256),
                0, q, N, L, G, cnt);
  else
    WSIC_LAUNCH("rans_esc", 4.0 * (double)N, st, k_rans_esc_count<false>, dim3((unsigned)G),
                dim3(256), 0, q, N, L, G, cnt);
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
  if (nsym > 4096 || n_in <= 0 || n_in > 0x7fffffff) return WSIC_E_INVAL;
  const dim3 grid((unsigned)((G + DW - 1) / DW));
  const double work = (double)N * (mode == 0 ? 4.0 : (mode == 1 ? 4.0 : 2.0));
  const bool sl = n_in <= SL_COLS;
#define WSIC_RANS_DEC(M, S)                                                                        \
  WSIC_LAUNCH("rans_decode", work, st, (k_rans_decode<M, S>), grid, dim3(64 * DW), 0, freq, nsym, lo, \
              N, L, G, gofs, eofs, states, escapes, n_esc, payload, n_words, out, n_in, invd, c, flags)
  if (mode == 0) WSIC_RANS_DEC(0, false);
  else if (mode == 1 && sl) WSIC_RANS_DEC(1, true);
  else if (mode == 1) WSIC_RANS_DEC(1, false);
  else if (sl) WSIC_RANS_DEC(2, true);
  else WSIC_RANS_DEC(2, false);
#undef WSIC_RANS_DEC
  return WSIC_OK;
}

}  // namespace wsic
