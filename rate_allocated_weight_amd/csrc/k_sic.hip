// SIC kernels: successive interference cancellation inside one column block.
//
// In the scaled (Babai) form used on the device, with B_jk = U_jk / U_kk and y = U w^T,
//     z_j = y_j / c - sum_{k>j} B_jk q_k ,   q_j = rint(z_j),
// which equals t_j / Delta_j of the row form t_j = w_j + sum_{k>j} (U_jk/U_jj) e_k with
// Delta_j = c / U_jj (WaterSIC page, Sommario tecnico §2 items 1-2: reverse-order SIC,
// spacing inversely proportional to the Cholesky diagonal). The interference of columns to
// the right of the block arrives precomputed in G (an MFMA GEMM); this kernel does the
// sequential part: 128 columns, right to left, each rounded and fed into the block's
// remaining columns.
//
// Layout: a 256-thread workgroup takes 16 rows; the 16 lanes of a DPP row hold one weight
// row, lane l owning block columns l, l+16, ..., l+112 (8 fp64 targets in registers). The
// owner of column j rounds it, row_newbcast hands q_j to the other 15 lanes, and every lane
// subtracts B_ij q_j from its pending targets. The 128 steps are unrolled at compile time, so
// register indices and LDS offsets are constants.
//
// B's diagonal blocks are packed once per factor U (they do not depend on c): column j of a
// block keeps rows 0 .. 16*(j/16+1)-1, zero from row j on, so that in step j every lane reads
// its entries unconditionally (a zero leaves finished targets unchanged). Columns go in pairs
// (2m+1, 2m), which share their row count: the pair starts at 16 (a+1)(8a + r) for its even
// column 2m = 16a + r, and row i of the pair holds the odd column's entry then the even one's,
// so one 16-byte LDS read serves two steps. A block holds 9216 doubles (72 KiB).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "pipe.h"

namespace wsic {
namespace {

constexpr int BW = 128;                  // block width
constexpr int HIT_CAP = 32;              // decisions re-checked one by one before a full redo
constexpr int PACK = 9216;               // doubles per packed block
constexpr int pack_off(int j) { return 16 * ((j >> 4) + 1) * (8 * (j >> 4) + (j & 15)); }
static_assert(pack_off(BW) == PACK, "packed block size");

template <int L>
__device__ __forceinline__ double bcast_row(double v) {
  // row_newbcast:L -- lane L of each 16-lane DPP row to every lane of that row
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), 0x150 + L, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), 0x150 + L, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Integer-interference mode: for each of a lane's 8 columns, the bound on the error of the
// interference it received (int8 limb products: 2^e_j * sum|q| * 2^-P, twice the fixed-point
// rounding bound, which also covers the fp64 combination) and the interference itself, so that
// a rounding decision closer to a boundary than the bound can be re-derived exactly.
struct Guard {
  float bnd[8];  // the bound, rounded up to float
};

// x >= 0 to float, rounded up (a few instructions instead of the library's directed rounding)
__device__ __forceinline__ float f32_up(double x) {
  const float f = (float)x;
  return ((double)f < x) ? __int_as_float(__float_as_int(f) + 1) : f;
}

// Steps 2M+1 and 2M of the in-block recursion (M = 63 ... 0), then the remaining ones. Columns
// past the end of a ragged last block hold z = 0 and all-zero B entries, so their steps change
// nothing and need no branch. A column's target is final once its own step has run (later steps
// only touch columns left of it), so rounding decisions can be checked after the block.
//
// The B entries of a pair are read from LDS one pair ahead (bo, be: this pair's odd and even
// column, no, ne: the next pair's), and the target the next step rounds is updated first, so the
// sequential chain per column is round -> broadcast -> one FMA. bl points at the lane's first
// entry (two doubles per row and pair).
template <int M>
__device__ __forceinline__ void load_pair(double (&bo)[8], double (&be)[8],
                                          const double* __restrict__ bl) {
  if constexpr (M >= 0) {
    constexpr int a = (2 * M) >> 4, off = pack_off(2 * M);
#pragma unroll
    for (int sp = 0; sp <= a; ++sp) {
      const double2 v = *reinterpret_cast<const double2*>(bl + off + 32 * sp);
      bo[sp] = v.x;
      be[sp] = v.y;
    }
  }
}

// hook(integral_constant<J>) runs at the start of step J: the super-block kernel issues the next
// block's loads there, spread over the LDS-bound steps instead of in one burst.
struct NoHook {
  template <class T>
  __device__ __forceinline__ void operator()(T) const {}
};

// step J with B entries b (column J of the block)
template <int J, class H>
__device__ __forceinline__ void sic_step(double (&z)[8], const double (&b)[8], H& hook) {
  hook(std::integral_constant<int, J>{});
  constexpr int a = J >> 4, l = J & 15;
  constexpr int an = (J - 1) >> 4;  // group of the next step's target (a or a - 1)
  const double qb = bcast_row<l>(rint(z[a]));
  if constexpr (J > 0) z[an] = fma(-b[an], qb, z[an]);
#pragma unroll
  for (int sp = 0; sp <= a; ++sp)
    if (J == 0 || sp != an) z[sp] = fma(-b[sp], qb, z[sp]);
}

template <int M>
struct Pairs {
  template <class H>
  static __device__ __forceinline__ void run(double (&z)[8], const double* __restrict__ bl,
                                             const double (&bo)[8], const double (&be)[8], H& hook) {
    double no[8], ne[8];
    load_pair<M - 1>(no, ne, bl);
    sic_step<2 * M + 1>(z, bo, hook);
    sic_step<2 * M>(z, be, hook);
    Pairs<M - 1>::run(z, bl, no, ne, hook);
  }
};
template <>
struct Pairs<-1> {
  template <class H>
  static __device__ __forceinline__ void run(double (&)[8], const double*, const double (&)[8],
                                             const double (&)[8], H&) {}
};

// bl: the block's packed B plus 2 * (lane within its DPP row)
template <class H = NoHook>
__device__ __forceinline__ void run_block(double (&z)[8], const double* __restrict__ bl,
                                          H&& hook = H{}) {
  double bo[8], be[8];
  load_pair<BW / 2 - 1>(bo, be, bl);
  Pairs<BW / 2 - 1>::run(z, bl, bo, be, hook);
}

// I8 = the interference G came from the int8 limb product (k_limb.hip): then the leaf also
// applies the exact excess of codes beyond +-127 listed by earlier leaves, guards its rounding
// decisions with the error bound, and emits what the next limb products need: the int8 code
// plane, the row sums of |q| and its own excess list.
template <bool HAS_G, bool HAS_RESID, bool I8, bool FUSE>
__global__ __launch_bounds__(256) void k_sic_leaf(LeafArgs p) {
  static_assert(!FUSE || I8, "the fused product is the int8 one");
  constexpr bool GIN = HAS_G || FUSE;  // the block receives interference from finished columns
  __shared__ __attribute__((aligned(16))) double Bs[PACK];
  const int tid = threadIdx.x;
  const int l16 = tid & 15, lane = tid & 63;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool active = row < p.n_out;
  const int64_t j0 = p.j0;
  const int w = p.w;

  // Every global load of the prologue is issued before the first is used: the per-row and
  // per-column operands, then the packed B block (all 18 16-byte loads of a thread in flight
  // before its LDS stores).
  double S = 0.0;  // sum of |q| over the columns right of this block (I8 mode)
  int cnt0 = 0;    // entries in this row's excess list so far (I8 mode)
  if (I8 && active) {
    S = p.absq[row];
    cnt0 = p.ocnt[row];
  }
  double yv[8], gv[8], bsc[8], dsc[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int j = l16 + 16 * s;
    const bool in = active && j < w;
    yv[s] = in ? p.Y[row * p.ldy + j0 + j] : 0.0;
    gv[s] = (HAS_G && in) ? p.G[row * p.ldg + j0 + j] : 0.0;
    bsc[s] = (I8 && GIN && in) ? p.bscale[j0 + j] : 0.0;
    dsc[s] = (HAS_RESID && in) ? p.invd[j0 + j] : 0.0;
  }
  // Interference of the finished columns [kf0, kf0 + kf) next to the block, formed here on the
  // int8 matrix cores (the same digit planes and error bound as the separate product): wave v
  // takes block columns 32 v .. 32 v + 31 against the workgroup's 16 rows (a 32-row fragment with
  // the upper half zero), 5 digit accumulators, combined in fp64 and staged through LDS (the
  // B-block area, loaded afterwards) into the target layout.
  double fz[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) fz[s] = 0.0;
  if constexpr (FUSE) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    typedef int v16i __attribute__((ext_vector_type(16)));
    const int wv = tid >> 6, mrow = lane & 31, kh = lane >> 5;
    const int64_t arow = (int64_t)blockIdx.x * 16 + mrow;
    const bool a_ok = mrow < 16 && arow < p.n_out;
    const int jn = 32 * wv + (lane & 31);
    const bool b_ok = jn < w;
    const int8_t* ap = p.q8 + (a_ok ? arow : 0) * p.ldq8 + p.kf0 + 16 * kh;
    const int8_t* bp = p.D + (j0 + (b_ok ? jn : 0)) * p.ldd + p.kf0 + 16 * kh;
    const int nks = (p.kf + 31) / 32;
    v16i acc[LIMBS];
#pragma unroll
    for (int l = 0; l < LIMBS; ++l) acc[l] = (v16i){};
    // k-steps in groups of GK: every operand load of a group is in flight before its products
    constexpr int GK = 4;
    for (int k0 = 0; k0 < nks; k0 += GK) {
      v4i a[GK], b[GK][LIMBS];
#pragma unroll
      for (int g4 = 0; g4 < GK; ++g4) {
        const bool in = k0 + g4 < nks;
        a[g4] = (a_ok && in) ? *reinterpret_cast<const v4i*>(ap + 32 * (k0 + g4)) : (v4i){0, 0, 0, 0};
#pragma unroll
        for (int l = 0; l < LIMBS; ++l)
          b[g4][l] = (b_ok && in) ? *reinterpret_cast<const v4i*>(bp + l * p.plane + 32 * (k0 + g4))
                                  : (v4i){0, 0, 0, 0};
      }
#pragma unroll
      for (int g4 = 0; g4 < GK; ++g4)
#pragma unroll
        for (int l = 0; l < LIMBS; ++l)
          acc[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[g4], b[g4][l], acc[l], 0, 0, 0);
    }
    const double es = b_ok ? p.escale[j0 + jn] : 0.0;
    double* Fs = Bs;  // [16][BW]
#pragma unroll
    for (int r = 0; r < 8; ++r) {  // result rows 8 (r/4) + 4 kh + r%4 < 16
      double f = 0.0;
#pragma unroll
      for (int l = 0; l < LIMBS; ++l)
        f = fma((double)acc[l][r], ldexp(1.0, 8 * (LIMBS - 1 - l)), f);
      Fs[(8 * (r >> 2) + 4 * kh + (r & 3)) * BW + jn] = f * es;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) fz[s] = Fs[(tid >> 4) * BW + l16 + 16 * s];
    __syncthreads();  // before the B block overwrites the staging area
  }
  {
    constexpr int PER = PACK / 2 / 256;
    static_assert(PER * 256 * 2 == PACK, "packed block is a whole number of 16-byte rounds");
    const uint4* src = reinterpret_cast<const uint4*>(p.Bpk);
    uint4* dst = reinterpret_cast<uint4*>(Bs);
    uint4 v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = src[e * 256 + tid];
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e * 256 + tid] = v[e];
  }

  double z[8];
  Guard g;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    z[s] = yv[s] * p.invc - gv[s] - fz[s];
    g.bnd[s] = (I8 && GIN) ? __double2float_ru(bsc[s] * S * LIMB_EPS * p.guard_scale) : 0.0f;
  }
  if (I8 && GIN && active) {
    // exact interference of the excess of large codes to the right (fp64)
    const int cnt = min(cnt0, OCAP);
    for (int o = 0; o < cnt; ++o) {
      const int2 e = p.olist[row * OCAP + o];
      const double f = p.invd[e.x] * (double)e.y;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = l16 + 16 * s;
        if (j < w) z[s] -= p.U[(j0 + j) * p.ldu + e.x] * f;
      }
    }
  }
  // incoming interference as received (int8 product + exact excess terms), for the check below
  double gin[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) gin[s] = yv[s] * p.invc - z[s];
  __syncthreads();

  run_block(z, Bs + 2 * l16);
  if (I8 && GIN) {
    // A rounding decision closer to a boundary than the error bound of the int8 product is
    // first re-checked on its own: the workgroup forms that decision's exact fp64 interference
    // (one dot product over the finished columns, split over all 256 threads) and compares the
    // rounding. Only when some decision would change (or there are too many to check) is the
    // whole block re-derived from exact interference.
    __shared__ int n_hit, must_redo;
    __shared__ int hit_j[HIT_CAP];
    __shared__ int hit_r[HIT_CAP];
    __shared__ double hit_z[HIT_CAP], hit_g[HIT_CAP];
    __shared__ double red[4];
    if (tid == 0) {
      n_hit = 0;
      must_redo = 0;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (0.5 - fabs(z[s] - rint(z[s])) <= (double)g.bnd[s]) {
        const int h = atomicAdd(&n_hit, 1);
        if (h < HIT_CAP) {
          hit_j[h] = l16 + 16 * s;
          hit_r[h] = tid >> 4;
          hit_z[h] = z[s];
          hit_g[h] = gin[s];
        }
      }
    }
    __syncthreads();
    const int nh = n_hit;
    if (tid == 0 && nh > 0) atomicAdd(p.flags + 2, nh);  // count of re-checked decisions
    if (nh > HIT_CAP) {
      if (tid == 0) must_redo = 1;
    } else {
      const int64_t kbeg = j0 + BW;
      for (int h = 0; h < nh; ++h) {
        const int64_t rr = (int64_t)blockIdx.x * 16 + hit_r[h];
        const double* ur = p.U + (j0 + hit_j[h]) * p.ldu;
        const int32_t* qr = p.codes + rr * p.ldq;
        double part = 0.0;
#pragma unroll 4
        for (int64_t k = kbeg + tid; k < p.n_in; k += 256)
          part = fma(ur[k], (double)qr[k] * p.invd[k], part);
        for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
        if (lane == 0) red[tid >> 6] = part;
        __syncthreads();
        if (tid == 0) {
          const double dot = (red[0] + red[1]) + (red[2] + red[3]);
          const double zx = hit_z[h] + (hit_g[h] - dot);
          if (rint(zx) != rint(hit_z[h])) must_redo = 1;
        }
        __syncthreads();
      }
    }
    __syncthreads();
    if (must_redo) {
      // each lane streams its own 8 rows of U along k in 4-column chunks (contiguous loads),
      // against its row's codes scaled by 1/U_kk
      const int64_t kbeg = j0 + BW;
      double acc[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) acc[s] = 0.0;
      if (active) {
        const int32_t* qrow = p.codes + row * p.ldq;
        constexpr int CH = 4;
        const int64_t kfull = kbeg + ((p.n_in - kbeg) / CH) * CH;
#pragma unroll 1
        for (int64_t k = kbeg; k < kfull; k += CH) {
          double qk[CH];
#pragma unroll
          for (int e = 0; e < CH; ++e) qk[e] = (double)qrow[k + e] * p.invd[k + e];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int j = l16 + 16 * s;
            if (j < w) {
              const double* ur = p.U + (j0 + j) * p.ldu + k;
#pragma unroll
              for (int e = 0; e < CH; ++e) acc[s] = fma(ur[e], qk[e], acc[s]);
            }
          }
        }
        for (int64_t k = kfull; k < p.n_in; ++k) {
          const double q = (double)qrow[k] * p.invd[k];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int j = l16 + 16 * s;
            if (j < w) acc[s] = fma(p.U[(j0 + j) * p.ldu + k], q, acc[s]);
          }
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = l16 + 16 * s;
        z[s] = (active && j < w) ? yv[s] * p.invc - acc[s] : 0.0;
      }
      if (tid == 0) atomicAdd(p.flags + 1, 1);  // count of exact re-derivations
      run_block(z, Bs + 2 * l16);
    }
  }

  int bad = 0;
  double asum = 0.0;
  int nexc = 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int j = l16 + 16 * s;
    if (active && j < w) {
      const double q = rint(z[s]);
      int32_t qi = 0;
      if (q >= -2147483647.0 && q <= 2147483647.0) {
        qi = (int32_t)q;
      } else {
        bad |= (z[s] == z[s]) ? FLAG_RANGE : FLAG_NONFINITE;
      }
      p.codes[row * p.ldq + j0 + j] = qi;
      if (HAS_RESID) p.resid[row * p.ldr + j0 + j] = (float)((z[s] - q) * (p.c * dsc[s]));
      if (I8) {
        const int q8 = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
        p.q8[row * p.ldq8 + j0 + j] = (int8_t)q8;
        asum += fabs(q);
        nexc += (q8 != qi);
      }
    }
  }
  if (I8) {
    // row totals over the 16 lanes; deterministic order of the excess list (lane, then slot)
    double tot = asum;
    int ntot = nexc;
    for (int m = 8; m >= 1; m >>= 1) {
      tot += __shfl_xor(tot, m, 16);
      ntot += __shfl_xor(ntot, m, 16);
    }
    int pre = nexc;  // inclusive scan of nexc over lanes 0..l16
    for (int d = 1; d < 16; d <<= 1) {
      const int t = __shfl_up(pre, d, 16);
      if (l16 >= d) pre += t;
    }
    pre -= nexc;
    const int base = cnt0;
    if (active && nexc) {
      int idx = base + pre;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = l16 + 16 * s;
        if (j < w) {
          const int32_t qi = p.codes[row * p.ldq + j0 + j];
          const int q8 = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
          if (q8 != qi) {
            if (idx < OCAP)
              p.olist[row * OCAP + idx] = make_int2((int)(j0 + j), qi - q8);
            else
              bad |= FLAG_OVERFLOW_LIST;
            ++idx;
          }
        }
      }
    }
    if (active && l16 == 0) {
      p.absq[row] = S + tot;
      p.ocnt[row] = base + ntot;
    }
  }
  if (bad) atomicOr(p.flags, bad);
}

// ------------------------------------------------------------------ super-block kernel
// With the int8 product, up to SUP_BLOCKS blocks of 128 columns [lo, hi) are finished by one
// launch: each workgroup walks its 16 rows through the blocks right to left. For every block it
// forms the interference of the super-block's finished columns on the int8 matrix cores from its
// own codes (kept in LDS) and the digit planes, runs the 128 sequential steps as the leaf does,
// checks its rounding decisions against the error bound, and writes codes, residuals, int8 codes
// and excess entries. While a block's steps run, the next block's packed B (global -> LDS,
// second buffer) and its Y / G / scale operands (registers) are already on the way. Row sums
// and list counts stay in registers across the blocks.
constexpr int SUP_BLOCKS = 4;  // matches the recursion's super-block width
constexpr int SUP_W = SUP_BLOCKS * BW;
constexpr int SUP_RING = 4;  // 4 KiB units of the fused product in flight per wave
static_assert(4 * SUP_RING * 4096 <= PACK * 8, "product rings fit the idle buffer");
constexpr int PACK_DMA = PACK * 8 / 1024 / 4;  // 16-byte direct LDS loads per wave per block
static_assert(PACK_DMA * 4 * 1024 == PACK * 8, "packed block is a whole number of 1 KiB rounds");

template <bool HAS_G, bool HAS_RESID>
__global__ __launch_bounds__(256) void k_sic_super(LeafArgs p) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  typedef int v16i __attribute__((ext_vector_type(16)));
  // two packed-B buffers as separate objects, so that the compiler can tell the prefetch into
  // one from the reads of the other (the loop below is unrolled by two for that)
  __shared__ __attribute__((aligned(1024))) double BsA[PACK];
  __shared__ __attribute__((aligned(1024))) double BsB[PACK];
  // (rows padded by 16 bytes: the 16 rows an operand read touches then sit on different banks)
  __shared__ __attribute__((aligned(16))) int8_t q8s[16][SUP_W + 16];
  __shared__ int n_hit, must_redo;
  __shared__ int hit_j[HIT_CAP];
  __shared__ int hit_r[HIT_CAP];
  __shared__ double hit_z[HIT_CAP], hit_g[HIT_CAP];
  __shared__ double red[4];

  const int tid = threadIdx.x;
  const int l16 = tid & 15, lane = tid & 63, wave = tid >> 6;
  const int rloc = tid >> 4;
  const int64_t row = (int64_t)blockIdx.x * 16 + rloc;
  const bool active = row < p.n_out;
  const int64_t rowc = active ? row : 0;  // clamped row for unconditional loads
  const int64_t lo = p.j0, hi = p.j0 + p.w;
  const int nb = (p.w + BW - 1) / BW;

  // this workgroup's int8 codes of the range (zero past hi)
  for (int e = tid; e < 16 * (SUP_W + 16) / 16; e += 256)
    reinterpret_cast<uint4*>(&q8s[0][0])[e] = make_uint4(0, 0, 0, 0);

  double S = 0.0;  // sum of |q| over the finished columns of this row
  int cnt = 0;     // entries in this row's excess list
  if (active) {
    S = p.absq[row];
    cnt = p.ocnt[row];
  }
  int bad = 0;

  // block b's packed B into LDS buffer `buf`; its per-row / per-column operands into registers
  auto issue_pack = [&](int b, double* buf) {
    const char* src = reinterpret_cast<const char*>(p.Bpk + (lo / BW + b) * PACK);
    char* dst = reinterpret_cast<char*>(buf);
#pragma unroll
    for (int i = 0; i < PACK_DMA; ++i) {
      const int ins = PACK_DMA * wave + i;
      pipe::dma16(src + 1024 * ins + 16 * lane, dst + 1024 * ins);
    }
  };
  auto load_ops = [&](int b, double (&yv)[8], double (&gv)[8], double (&bsc)[8], double (&dv)[8]) {
    const int64_t j0 = lo + (int64_t)b * BW;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t jc = j0 + l16 + 16 * s < hi ? j0 + l16 + 16 * s : hi - 1;  // clamped column
      yv[s] = p.Y[rowc * p.ldy + jc];
      gv[s] = HAS_G ? p.G[rowc * p.ldg + jc] : 0.0;
      bsc[s] = p.bscale[jc];
      dv[s] = HAS_RESID ? p.invd[jc] : 0.0;
    }
  };

  // Y, G, the bound's column scale (rounded up to float) and 1/U_jj (for the residuals) of the
  // current block. (1/U_jj is loaded ahead too: read in the output loop, behind its stores, each
  // load would wait for the stores before it.)
  double yv[8], gv[8], dv[8];
  float bsf[8];
  {
    double b0[8];
    issue_pack(nb - 1, BsA);
    load_ops(nb - 1, yv, gv, b0, dv);
#pragma unroll
    for (int s = 0; s < 8; ++s) bsf[s] = f32_up(b0[s]);
  }

  auto do_block = [&](int b, double* Bcur, double* Bidle) {
    const int64_t j0 = lo + (int64_t)b * BW;
    const int w = (int)(hi - j0 < BW ? hi - j0 : BW);
    // the check's counters start at zero: every read of them in the previous block precedes its
    // closing barrier, and the barriers before this block's check order the reset before it
    if (tid == 0) {
      n_hit = 0;
      must_redo = 0;
    }
    const int64_t kf0 = j0 + BW;
    const int kf = (int)(hi - kf0);  // finished columns of the range right of this block
    const bool gin = HAS_G || kf > 0;

    // interference of the range's finished columns [kf0, hi) (int8 product, as in the leaf)
    double fz[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) fz[s] = 0.0;
    if (kf > 0) {  // uniform
      const int mrow = lane & 31, kh = lane >> 5;
      const int jn = 32 * wave + (lane & 31);
      const bool b_ok = jn < w;
      const int8_t* as = &q8s[mrow & 15][(int)(kf0 - lo) + 16 * kh];
      // The digit planes stream through a per-wave ring of SUP_RING units in the idle buffer; a
      // unit is one plane over 4 k-steps: 32 rows x 128 bytes, fetched as whole cache lines (8
      // lanes per row) by 4 direct loads. Chunk c of row r sits at 16-byte slot 8 r + (c ^ r%8),
      // so an MFMA operand read (32 rows, one chunk) touches every LDS bank once.
      const int nq = (kf + 127) / 128;  // k-quads (rows are zero-padded to whole lines)
      const int nu = nq * LIMBS;
      char* ring = reinterpret_cast<char*>(Bidle) + wave * (SUP_RING * 4096);
      // (a block with finished columns to its right in the range is a whole 128 columns wide)
      const int8_t* brow = p.D + (j0 + 32 * wave) * p.ldd + kf0;
      auto issue_u = [&](int u) {
        const int q = u / LIMBS, l = u - q * LIMBS;
        char* slot = ring + (u % SUP_RING) * 4096;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * i + (lane >> 3);
          const int c = (lane & 7) ^ (r & 7);
          pipe::dma16(brow + l * p.plane + r * p.ldd + 128 * q + 16 * c, slot + 1024 * i);
        }
      };
      // this lane's operand slots for the 4 k-steps of a unit (row mrow, chunk 2 t + kh)
      unsigned ro[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) ro[t] = 16u * (8 * mrow + ((2 * t + kh) ^ (mrow & 7)));
      v16i acc[LIMBS];
#pragma unroll
      for (int l = 0; l < LIMBS; ++l) acc[l] = (v16i){};
#pragma unroll
      for (int u = 0; u < SUP_RING; ++u)
        if (u < nu) issue_u(u);
#pragma unroll 1
      for (int q = 0; q < nq; ++q) {
        // this quad's A operands (the workgroup's codes; rows 16-31 of the fragment are zero),
        // read in assembly for the same reason as the ring below
        v4i a[4];
        const unsigned sa = (unsigned)reinterpret_cast<uintptr_t>((const pipe::lds_char*)(as + 128 * q));
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %4 offset:32\n\t"
            "ds_read_b128 %2, %4 offset:64\n\t"
            "ds_read_b128 %3, %4 offset:96\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
            : "v"(sa)
            : "memory");
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (mrow >= 16) a[t] = (v4i){0, 0, 0, 0};
        // planes in pairs (two independent accumulation chains interleaved), the fifth alone
#pragma unroll
        for (int l = 0; l < LIMBS; l += 2) {
          const int u = q * LIMBS + l;
          const bool two = l + 1 < LIMBS;
          const int ul = two ? u + 1 : u;  // the last unit this step needs
          // units issued so far: 0 .. u + SUP_RING - 1, so after ul the ring holds
          // SUP_RING - 2 (pair) or SUP_RING - 1 (single) more, fewer at the end
          pipe::wait_ahead<4, SUP_RING - 1>(min(nu - 1 - ul, two ? SUP_RING - 2 : SUP_RING - 1));
          // read in assembly with its wait inside: the compiler would otherwise order every
          // read of this buffer behind all direct loads in flight
          const unsigned sb0 =
              (unsigned)reinterpret_cast<uintptr_t>((const pipe::lds_char*)(ring + (u % SUP_RING) * 4096));
          v4i b0[4], b1[4];
          if (two) {
            const unsigned sb1 = (unsigned)reinterpret_cast<uintptr_t>(
                (const pipe::lds_char*)(ring + ((u + 1) % SUP_RING) * 4096));
            asm volatile(
                "ds_read_b128 %0, %8\n\t"
                "ds_read_b128 %1, %9\n\t"
                "ds_read_b128 %2, %10\n\t"
                "ds_read_b128 %3, %11\n\t"
                "ds_read_b128 %4, %12\n\t"
                "ds_read_b128 %5, %13\n\t"
                "ds_read_b128 %6, %14\n\t"
                "ds_read_b128 %7, %15\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(b0[0]), "=&v"(b0[1]), "=&v"(b0[2]), "=&v"(b0[3]),
                  "=&v"(b1[0]), "=&v"(b1[1]), "=&v"(b1[2]), "=&v"(b1[3])
                : "v"(sb0 + ro[0]), "v"(sb0 + ro[1]), "v"(sb0 + ro[2]), "v"(sb0 + ro[3]),
                  "v"(sb1 + ro[0]), "v"(sb1 + ro[1]), "v"(sb1 + ro[2]), "v"(sb1 + ro[3])
                : "memory");
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              acc[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], b0[t], acc[l], 0, 0, 0);
              acc[l + 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], b1[t], acc[l + 1], 0, 0, 0);
            }
            // the two slots' operands are in registers
            if (u + SUP_RING < nu) issue_u(u + SUP_RING);
            if (u + 1 + SUP_RING < nu) issue_u(u + 1 + SUP_RING);
          } else {
            asm volatile(
                "ds_read_b128 %0, %4\n\t"
                "ds_read_b128 %1, %5\n\t"
                "ds_read_b128 %2, %6\n\t"
                "ds_read_b128 %3, %7\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(b0[0]), "=&v"(b0[1]), "=&v"(b0[2]), "=&v"(b0[3])
                : "v"(sb0 + ro[0]), "v"(sb0 + ro[1]), "v"(sb0 + ro[2]), "v"(sb0 + ro[3])
                : "memory");
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[t], b0[t], acc[l], 0, 0, 0);
            if (u + SUP_RING < nu) issue_u(u + SUP_RING);
          }
        }
      }
      pipe::barrier_lds();  // every wave done with its ring before the staging overwrites it
      const double es = b_ok ? p.escale[j0 + jn] : 0.0;
#pragma unroll
      for (int r = 0; r < 8; ++r) {  // result rows 8 (r/4) + 4 kh + r%4 < 16
        double f = 0.0;
#pragma unroll
        for (int l = 0; l < LIMBS; ++l)
          f = fma((double)acc[l][r], ldexp(1.0, 8 * (LIMBS - 1 - l)), f);
        Bidle[(8 * (r >> 2) + 4 * kh + (r & 3)) * BW + jn] = f * es;
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 8; ++s) fz[s] = Bidle[rloc * BW + l16 + 16 * s];
    }
    // this block's packed B has landed (issued during the previous block); the idle buffer is
    // free once every wave has read the staging
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    double z[8], gin_v[8];
    Guard g;
    // the bound S 2^-P (guard scale) per row, rounded up; times the column scale and a margin
    // that covers the float product's rounding
    const float tb = f32_up(S * LIMB_EPS * p.guard_scale) * (1.0f + 0x1p-22f);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int j = l16 + 16 * s;
      const bool in = active && j < w;
      const double zv = yv[s] * p.invc - gv[s] - fz[s];
      z[s] = in ? zv : 0.0;
      g.bnd[s] = (in && gin) ? tb * bsf[s] : 0.0f;
    }
    {
      // Exact interference of the excess of large codes to the right (fp64); the list may have
      // grown in this launch, so its entries are read past the L1 cache. The loop runs to the
      // longest list of the wave with every lane's own terms predicated (clamped loads, zero
      // factors), so that no divergent branch opens here: the compiler has been seen to place
      // register copies in the join block of such a branch ahead of its exec-mask restore, which
      // leaves them unwritten in the lanes that skipped it (checked in the assembly at build).
      const int my_cn = active ? min(cnt, OCAP) : 0;
      int cn = 0;
      if (__ballot(my_cn > 0) != 0) {  // uniform; usually no row of the wave has a list
        cn = my_cn;
        for (int m = 32; m >= 1; m >>= 1) cn = max(cn, __shfl_xor(cn, m, 64));
        cn = __builtin_amdgcn_readfirstlane(cn);
      }
      const long long* ol = reinterpret_cast<const long long*>(p.olist + rowc * OCAP);
      for (int o = 0; o < cn; ++o) {
        const bool use = o < my_cn;
        const long long raw =
            __hip_atomic_load(ol + (use ? o : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int ex = use ? (int)(raw & 0xffffffffll) : (int)lo;  // lo: any valid column
        const double f = use ? p.invd[ex] * (double)(int)(raw >> 32) : 0.0;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int j = l16 + 16 * s;
          const int64_t jr = j0 + (j < w ? j : 0);
          const double t = p.U[jr * p.ldu + ex] * f;
          z[s] = (j < w) ? z[s] - t : z[s];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) gin_v[s] = yv[s] * p.invc - z[s];
    // The next block's loads are issued during this block's steps (LDS-bound, so the memory
    // instructions fill idle issue slots instead of stalling in one burst): the L2 warm-up of
    // its digit planes (each 128-byte line touched by one thread of the workgroups that share an
    // L2; workgroups are dealt to the 8 XCDs round-robin) at the first step, its packed B
    // (PACK_DMA direct loads per wave) every 3 steps, its Y, G and column scales (one register
    // each) every 6 steps, all in the first half so they have landed by the end of the block.
    // They are issued after this block's own loads above: the memory counter completes in
    // order.
    // (No branches in the hook: after the last block of the launch it reloads this block's
    // operands into the idle buffer and registers, which nothing reads.)
    double yn[8], gn[8], bn[8], dn[8];
    int pf = 0;  // touched digit-plane words (consumed below, never used)
    const int64_t jn0 = b > 0 ? j0 - BW : j0;  // the next block
    auto hook = [&](auto Jc) __attribute__((always_inline)) {
      constexpr int J = decltype(Jc)::value;
      if constexpr (J == BW - 1) {
        // line i: row i % 128 of the next block, plane (i / 128) % 5, line (i / 128) / 5 of the
        // row's bytes [j0, hi); at most two per thread, out-of-range indices clamped
        const int nlr = (int)((hi - j0 + 127) / 128);
        const int nl = LIMBS * BW * nlr;
        const int per_xcd = (int)((gridDim.x + 7 - (blockIdx.x & 7)) / 8);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          int i = ((int)(blockIdx.x >> 3) + it * per_xcd) * 256 + tid;
          i = i < nl ? i : nl - 1;
          const int r = i & (BW - 1), t = i >> 7, c = t / LIMBS, l = t - LIMBS * c;
          const int64_t row_d = jn0 + r < hi ? jn0 + r : hi - 1;  // a ragged block's rows end at hi
          pf ^= *reinterpret_cast<const int*>(p.D + l * p.plane + row_d * p.ldd + j0 + 128 * c);
        }
      }
      constexpr int dj = BW - 2 - J;
      if constexpr (dj >= 0 && dj % 3 == 0 && dj / 3 < PACK_DMA) {
        const char* src = reinterpret_cast<const char*>(p.Bpk + (jn0 / BW) * PACK);
        const int ins = PACK_DMA * wave + dj / 3;
        pipe::dma16(src + 1024 * ins + 16 * lane, reinterpret_cast<char*>(Bidle) + 1024 * ins);
      }
      constexpr int oj = BW - 3 - J;
      if constexpr (oj >= 0 && oj % 6 == 0 && oj / 6 < 8) {
        constexpr int sv = oj / 6;
        const int64_t jc = jn0 + l16 + 16 * sv;
        const int64_t jcc = jc < hi ? jc : hi - 1;  // (the last block of the matrix may be ragged)
        yn[sv] = p.Y[rowc * p.ldy + jcc];
        gn[sv] = HAS_G ? p.G[rowc * p.ldg + jcc] : 0.0;
        bn[sv] = p.bscale[jcc];
        dn[sv] = HAS_RESID ? p.invd[jcc] : 0.0;
      }
    };

    // the lane's offset is made opaque here so that the block's LDS addresses are formed inside
    // the loop (immediate offsets) instead of being hoisted into hundreds of live registers
    int lb = 2 * l16;
    asm volatile("" : "+v"(lb));
    run_block(z, Bcur + lb, hook);

    if (gin) {  // uniform
      // decisions inside the error bound: re-check one by one, re-derive the block if needed
      // (LDS-only barriers: the next block's loads in flight need not land here)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (0.5 - fabs(z[s] - rint(z[s])) <= (double)g.bnd[s]) {
          const int h = atomicAdd(&n_hit, 1);
          if (h < HIT_CAP) {
            hit_j[h] = l16 + 16 * s;
            hit_r[h] = rloc;
            hit_z[h] = z[s];
            hit_g[h] = gin_v[s];
          }
        }
      }
      pipe::barrier_lds();
      const int nh = n_hit;  // uniform: read after the barrier by every thread
      if (tid == 0 && nh > 0) atomicAdd(p.flags + 2, nh);
      // the re-check reads codes other waves stored in earlier blocks: fenced barrier first
      if (nh > 0) __syncthreads();
      if (nh > HIT_CAP) {
        if (tid == 0) must_redo = 1;
      } else {
        for (int h = 0; h < nh; ++h) {
          const int64_t rr = (int64_t)blockIdx.x * 16 + hit_r[h];
          const double* ur = p.U + (j0 + hit_j[h]) * p.ldu;
          const int32_t* qr = p.codes + rr * p.ldq;
          double part = 0.0;
#pragma unroll 4
          for (int64_t k = kf0 + tid; k < p.n_in; k += 256)
            part = fma(ur[k], (double)qr[k] * p.invd[k], part);
          for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
          if (lane == 0) red[wave] = part;
          __syncthreads();
          if (tid == 0) {
            const double dot = (red[0] + red[1]) + (red[2] + red[3]);
            const double zx = hit_z[h] + (hit_g[h] - dot);
            if (rint(zx) != rint(hit_z[h])) must_redo = 1;
          }
          __syncthreads();
        }
      }
      // must_redo is only ever set after hits; with none it is still the block's reset value
      if (nh > 0) pipe::barrier_lds();
      if (nh > 0 && must_redo) {
        double acc[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[s] = 0.0;
        if (active) {
          const int32_t* qrow = p.codes + row * p.ldq;
          constexpr int CH = 4;
          const int64_t kfull = kf0 + ((p.n_in - kf0) / CH) * CH;
#pragma unroll 1
          for (int64_t k = kf0; k < kfull; k += CH) {
            double qk[CH];
#pragma unroll
            for (int e = 0; e < CH; ++e) qk[e] = (double)qrow[k + e] * p.invd[k + e];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int j = l16 + 16 * s;
              if (j < w) {
                const double* ur = p.U + (j0 + j) * p.ldu + k;
#pragma unroll
                for (int e = 0; e < CH; ++e) acc[s] = fma(ur[e], qk[e], acc[s]);
              }
            }
          }
          for (int64_t k = kfull; k < p.n_in; ++k) {
            const double q = (double)qrow[k] * p.invd[k];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int j = l16 + 16 * s;
              if (j < w) acc[s] = fma(p.U[(j0 + j) * p.ldu + k], q, acc[s]);
            }
          }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int j = l16 + 16 * s;
          z[s] = (active && j < w) ? yv[s] * p.invc - acc[s] : 0.0;
        }
        if (tid == 0) atomicAdd(p.flags + 1, 1);
        run_block(z, Bcur + lb);
      }
    }

    asm volatile("" ::"v"(pf));  // the warming loads have long landed here
    // outputs of the block
    double asum = 0.0;
    int nexc = 0;
    int32_t qv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int j = l16 + 16 * s;
      qv[s] = 0;
      if (active && j < w) {
        const double q = rint(z[s]);
        int32_t qi = 0;
        if (q >= -2147483647.0 && q <= 2147483647.0) {
          qi = (int32_t)q;
        } else {
          bad |= (z[s] == z[s]) ? FLAG_RANGE : FLAG_NONFINITE;
        }
        qv[s] = qi;
        p.codes[row * p.ldq + j0 + j] = qi;
        if (HAS_RESID) p.resid[row * p.ldr + j0 + j] = (float)((z[s] - q) * (p.c * dv[s]));
        const int q8 = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
        p.q8[row * p.ldq8 + j0 + j] = (int8_t)q8;
        q8s[rloc][(int)(j0 - lo) + j] = (int8_t)q8;
        asum += fabs(q);
        nexc += (q8 != qi);
      }
    }
    double tot = asum;
    int ntot = nexc;
    for (int m = 8; m >= 1; m >>= 1) {
      tot += __shfl_xor(tot, m, 16);
      ntot += __shfl_xor(ntot, m, 16);
    }
    int pre = nexc;
    for (int d = 1; d < 16; d <<= 1) {
      const int t = __shfl_up(pre, d, 16);
      if (l16 >= d) pre += t;
    }
    pre -= nexc;
    if (active && nexc) {
      int idx = cnt + pre;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = l16 + 16 * s;
        if (j < w) {
          const int q8 = qv[s] > 127 ? 127 : (qv[s] < -127 ? -127 : qv[s]);
          if (q8 != qv[s]) {
            if (idx < OCAP)
              p.olist[row * OCAP + idx] = make_int2((int)(j0 + j), qv[s] - q8);
            else
              bad |= FLAG_OVERFLOW_LIST;
            ++idx;
          }
        }
      }
    }
    S += tot;
    cnt += ntot;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      yv[s] = yn[s];
      gv[s] = gn[s];
      bsf[s] = f32_up(bn[s]);
      dv[s] = dn[s];
    }
    // int8 codes in LDS visible to every wave; every wave done with this block's packed B
    // before it becomes the idle buffer. (Global stores are not waited for here: the next
    // block's reads of codes by other waves come after a fenced barrier, and a wave's own
    // excess entries are read after its wait for the packed B.)
    pipe::barrier_lds();
  };
  for (int b = nb - 1; b >= 0; b -= 2) {
    do_block(b, BsA, BsB);
    if (b >= 1) do_block(b - 1, BsB, BsA);
  }
  if (active && l16 == 0) {
    p.absq[row] = S;
    p.ocnt[row] = cnt;
  }
  if (bad) atomicOr(p.flags, bad);
}

// Packed diagonal blocks of B = U diag(1/U_jj): one block per 128 columns.
__global__ void k_pack_blocks(const double* __restrict__ U, int64_t ldu, int64_t n,
                              const double* __restrict__ invd, double* __restrict__ Bpk) {
  const int64_t blk = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;  // over 128 x 128
  if (e >= BW * BW) return;
  const int j = e / BW, i = e % BW;
  const int a = j >> 4;
  if (i >= 16 * (a + 1)) return;
  const int64_t j0 = blk * BW;
  double v = 0.0;
  if (i < j && j0 + j < n) v = U[(j0 + i) * ldu + j0 + j] * invd[j0 + j];
  Bpk[blk * PACK + pack_off(j & ~1) + 2 * i + (1 - (j & 1))] = v;  // odd column first
}

__global__ void k_prep(const double* U, int64_t ldu, int64_t n, double* invd, int* flags) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const double d = U[j * ldu + j];
  if (!(d > 0.0) || !isfinite(d)) {
    atomicOr(flags, FLAG_BAD_DIAG);
    invd[j] = 0.0;
    return;
  }
  invd[j] = 1.0 / d;
}

// Delta_j = c / U_jj (fp64 division, the step of column j) and the diagonal itself
__global__ void k_delta(const double* U, int64_t ldu, int64_t n, double c, double* delta,
                        double* diag) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const double d = U[j * ldu + j];
  if (delta) delta[j] = c / d;
  if (diag) diag[j] = d;
}

template <typename T>
__device__ __forceinline__ float elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float elem<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// a 32-bit word of two bf16 / one fp32 holds a NaN or Inf (all exponent bits set)
template <typename T>
__device__ __forceinline__ bool word_nonfinite(uint32_t w);
template <>
__device__ __forceinline__ bool word_nonfinite<uint16_t>(uint32_t w) {
  return (w & 0x7F80u) == 0x7F80u || (w & 0x7F800000u) == 0x7F800000u;
}
template <>
__device__ __forceinline__ bool word_nonfinite<float>(uint32_t w) {
  return (w & 0x7F800000u) == 0x7F800000u;
}

// Rows over the y dimension of the grid, each row's 16-byte chunks over x (VEC: rows start
// 16-byte aligned, checked by the launcher), the row's tail element by element.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_check_finite(const T* W, int64_t n_out, int64_t n_in,
                                                      int64_t ldw, int* flags) {
  constexpr int E = 16 / (int)sizeof(T);
  bool bad = false;
  const int64_t x0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t xs = (int64_t)gridDim.x * blockDim.x;
  const int64_t nv = VEC ? n_in / E : 0;
  for (int64_t r = blockIdx.y; r < n_out; r += gridDim.y) {
    const T* wr = W + r * ldw;
    if (VEC) {
      const uint4* v4 = reinterpret_cast<const uint4*>(wr);
      for (int64_t c = x0; c < nv; c += xs) {
        const uint4 v = v4[c];
        bad = bad || word_nonfinite<T>(v.x) || word_nonfinite<T>(v.y) ||
              word_nonfinite<T>(v.z) || word_nonfinite<T>(v.w);
      }
    }
    for (int64_t j = nv * E + x0; j < n_in; j += xs)
      if (!isfinite(elem<T>(wr, j))) bad = true;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, FLAG_NONFINITE);
}

// Column sums of W and W^2 over a slab of COLSTAT_ROWS rows: 256 columns (4 adjacent ones per
// thread, one 8- or 16-byte load per row when VEC) x 4 row lanes per workgroup, one partial pair
// per (slab, column); k_colstats_finish reduces the slabs in order. Every column's terms are
// summed in the same order whatever the load width.
constexpr int COLSTAT_ROWS = 64;
template <typename T>
struct Quad;
template <>
struct Quad<uint16_t> {
  typedef uint2 type;
  static __device__ __forceinline__ void get(const uint16_t* p, float (&v)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xFFFF0000u);
  }
};
template <>
struct Quad<float> {
  static __device__ __forceinline__ void get(const float* p, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  }
};
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_colstats(const T* W, int64_t n_out, int64_t n_in,
                                                  int64_t ldw, double* part,
                                                  const double* __restrict__ rs) {
  __shared__ double s1[4][256], s2[4][256];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 256 + 4 * tx;
  const int64_t r0 = (int64_t)blockIdx.y * COLSTAT_ROWS;
  double a[4] = {0.0, 0.0, 0.0, 0.0}, b[4] = {0.0, 0.0, 0.0, 0.0};
  const int64_t r1 = (r0 + COLSTAT_ROWS < n_out) ? r0 + COLSTAT_ROWS : n_out;
  if (VEC && j + 3 < n_in) {
    for (int64_t r = r0 + ty; r < r1; r += 4) {
      float v[4];
      Quad<T>::get(W + r * ldw + j, v);
      const double sc = rs ? rs[r] : 1.0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double x = rs ? (double)v[c] * sc : (double)v[c];
        a[c] += x;
        b[c] = fma(x, x, b[c]);
      }
    }
  } else {
    for (int64_t r = r0 + ty; r < r1; r += 4) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (j + c < n_in) {
          const double x = rs ? (double)elem<T>(W, r * ldw + j + c) * rs[r]
                              : (double)elem<T>(W, r * ldw + j + c);
          a[c] += x;
          b[c] = fma(x, x, b[c]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s1[ty][4 * tx + c] = a[c];
    s2[ty][4 * tx + c] = b[c];
  }
  __syncthreads();
  if (ty == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 4 * tx + c;
      if (j + c < n_in) {
        const double sa = (s1[0][t] + s1[1][t]) + (s1[2][t] + s1[3][t]);
        const double sb = (s2[0][t] + s2[1][t]) + (s2[2][t] + s2[3][t]);
        part[((int64_t)blockIdx.y * n_in + j + c) * 2 + 0] = sa;
        part[((int64_t)blockIdx.y * n_in + j + c) * 2 + 1] = sb;
      }
    }
  }
}

__global__ void k_colstats_finish(const double* part, int64_t n_out, int64_t n_in, int nslab,
                                  double* colvar) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_in) return;
  // slabs in order, their loads issued eight at a time
  double a = 0.0, b = 0.0;
  const double2* p2 = reinterpret_cast<const double2*>(part) + j;
  int s = 0;
  for (; s + 8 <= nslab; s += 8) {
    double2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p2[(int64_t)(s + u) * n_in];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a += v[u].x;
      b += v[u].y;
    }
  }
  for (; s < nslab; ++s) {
    const double2 v = p2[(int64_t)s * n_in];
    a += v.x;
    b += v.y;
  }
  const double mean = a / (double)n_out;
  const double v = b / (double)n_out - mean * mean;
  colvar[j] = v > 0.0 ? v : 0.0;
}

}  // namespace

int sic_pack_doubles(int64_t n_in) { return (int)((n_in + BW - 1) / BW) * PACK; }

int colstats_doubles(int64_t n_out, int64_t n_in) {
  return (int)(2 * n_in * ((n_out + COLSTAT_ROWS - 1) / COLSTAT_ROWS));
}

int launch_pack_blocks(const double* U, int64_t ldu, int64_t n, const double* invd, double* Bpk,
                       hipStream_t st) {
  const unsigned nblk = (unsigned)((n + BW - 1) / BW);
  WSIC_LAUNCH("pack_blocks", 8.0 * nblk * PACK, st, k_pack_blocks, dim3(BW * BW / 256, nblk),
              dim3(256), 0, U, ldu, n, invd, Bpk);
  return WSIC_OK;
}

int launch_sic_leaf(const LeafArgs& a, bool i8, hipStream_t st) {
  if (a.w <= 0 || a.w > BW || a.j0 % BW != 0) {
    set_error("internal: leaf at %lld width %d", (long long)a.j0, a.w);
    return WSIC_E_INVAL;
  }
  if (i8 && (!a.q8 || !a.absq || !a.ocnt || !a.olist || !a.U || !a.bscale)) {
    set_error("internal: integer-interference leaf without its buffers");
    return WSIC_E_INVAL;
  }
  if (a.kf > 0 && (!i8 || !a.D || !a.escale || a.kf0 != a.j0 + BW || (a.ldd % 16) != 0 ||
                   (a.ldq8 % 16) != 0 || (a.kf0 % 16) != 0)) {
    set_error("internal: fused leaf product preconditions");
    return WSIC_E_INVAL;
  }
  LeafArgs p = a;
  p.Bpk = a.Bpk + (a.j0 / BW) * PACK;
  p.invc = 1.0 / a.c;
  const unsigned blocks = (unsigned)((a.n_out + 15) / 16);
  // algorithmic bytes of the method's step: the weights in, the int32 codes out (the design's
  // intermediates -- Y, G, residuals, int8 codes -- are not counted)
  const double work = (double)a.n_out * a.w * (a.w_bytes + 4.0);
#define WSIC_LEAF(HG, HR, I8, FU)                                                                  \
  WSIC_LAUNCH("sic_leaf", work, st, (k_sic_leaf<HG, HR, I8, FU>), dim3(blocks), dim3(256), 0, p)
  const bool hg = a.G != nullptr, hr = a.resid != nullptr, fu = a.kf > 0;
  if (i8 && fu) {
    if (hg && hr) WSIC_LEAF(true, true, true, true);
    else if (hg) WSIC_LEAF(true, false, true, true);
    else if (hr) WSIC_LEAF(false, true, true, true);
    else WSIC_LEAF(false, false, true, true);
  } else if (i8) {
    if (hg && hr) WSIC_LEAF(true, true, true, false);
    else if (hg) WSIC_LEAF(true, false, true, false);
    else if (hr) WSIC_LEAF(false, true, true, false);
    else WSIC_LEAF(false, false, true, false);
  } else {
    if (hg && hr) WSIC_LEAF(true, true, false, false);
    else if (hg) WSIC_LEAF(true, false, false, false);
    else if (hr) WSIC_LEAF(false, true, false, false);
    else WSIC_LEAF(false, false, false, false);
  }
#undef WSIC_LEAF
  return WSIC_OK;
}

int launch_sic_super(const LeafArgs& a, hipStream_t st) {
  if (a.w <= 0 || a.w > SUP_W || a.j0 % BW != 0 || !a.q8 || !a.absq || !a.ocnt || !a.olist || !a.U ||
      !a.bscale || !a.D || !a.escale || (a.ldd % 16) != 0 || (a.ldq8 % 16) != 0) {
    set_error("internal: super-block launch at %lld width %d", (long long)a.j0, a.w);
    return WSIC_E_INVAL;
  }
  LeafArgs p = a;
  p.invc = 1.0 / a.c;
  const unsigned blocks = (unsigned)((a.n_out + 15) / 16);
  const double work = (double)a.n_out * a.w * (a.w_bytes + 4.0);  // as in launch_sic_leaf
  const bool hg = a.G != nullptr, hr = a.resid != nullptr;
  if (hg && hr)
    WSIC_LAUNCH("sic_leaf", work, st, (k_sic_super<true, true>), dim3(blocks), dim3(256), 0, p);
  else if (hg)
    WSIC_LAUNCH("sic_leaf", work, st, (k_sic_super<true, false>), dim3(blocks), dim3(256), 0, p);
  else if (hr)
    WSIC_LAUNCH("sic_leaf", work, st, (k_sic_super<false, true>), dim3(blocks), dim3(256), 0, p);
  else
    WSIC_LAUNCH("sic_leaf", work, st, (k_sic_super<false, false>), dim3(blocks), dim3(256), 0, p);
  return WSIC_OK;
}

int launch_prep(const double* U, int64_t ldu, int64_t n, double* invd, int* flags, hipStream_t st) {
  WSIC_LAUNCH("prep", 16.0 * n, st, k_prep, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, U,
              ldu, n, invd, flags);
  return WSIC_OK;
}

int launch_delta(const double* U, int64_t ldu, int64_t n, double c, double* delta, double* diag,
                 hipStream_t st) {
  WSIC_LAUNCH("delta", 16.0 * n, st, k_delta, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, U,
              ldu, n, c, delta, diag);
  return WSIC_OK;
}

int launch_check_finite(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                        int* flags, hipStream_t st) {
  if (n_out <= 0 || n_in <= 0) return WSIC_OK;
  const int64_t esz = dtype == WSIC_BF16 ? 2 : 4;
  const bool vec = (((uintptr_t)W) & 15) == 0 && (ldw * esz) % 16 == 0;
  const int64_t per_row = vec ? (n_in * esz + 15) / 16 : n_in;  // work items of a row
  const int64_t gx = std::min<int64_t>(std::max<int64_t>((per_row + 255) / 256, 1), 64);
  const int64_t gy = std::min<int64_t>(std::max<int64_t>(2048 / gx, 1), std::min<int64_t>(n_out, 65535));
  const dim3 grid((unsigned)gx, (unsigned)gy);
  const double work = (double)n_out * n_in * esz;
  if (dtype == WSIC_BF16) {
    if (vec)
      WSIC_LAUNCH("check_finite", work, st, (k_check_finite<uint16_t, true>), grid, dim3(256), 0,
                  (const uint16_t*)W, n_out, n_in, ldw, flags);
    else
      WSIC_LAUNCH("check_finite", work, st, (k_check_finite<uint16_t, false>), grid, dim3(256), 0,
                  (const uint16_t*)W, n_out, n_in, ldw, flags);
  } else {
    if (vec)
      WSIC_LAUNCH("check_finite", work, st, (k_check_finite<float, true>), grid, dim3(256), 0,
                  (const float*)W, n_out, n_in, ldw, flags);
    else
      WSIC_LAUNCH("check_finite", work, st, (k_check_finite<float, false>), grid, dim3(256), 0,
                  (const float*)W, n_out, n_in, ldw, flags);
  }
  return WSIC_OK;
}

int launch_colstats(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                    double* part, double* colvar, hipStream_t st, const double* rs) {
  if ((((uintptr_t)part) & 15) != 0) {
    set_error("internal: column partial sums not 16-byte aligned");
    return WSIC_E_INVAL;
  }
  const unsigned gx = (unsigned)((n_in + 255) / 256);
  const unsigned gy = (unsigned)((n_out + COLSTAT_ROWS - 1) / COLSTAT_ROWS);
  const int64_t esz = dtype == WSIC_BF16 ? 2 : 4;
  // 4-column loads need every row start aligned to 4 elements
  const bool vec = (((uintptr_t)W) & (4 * esz - 1)) == 0 && ldw % 4 == 0;
  const double work = (double)n_out * n_in * esz;
  if (dtype == WSIC_BF16) {
    if (vec)
      WSIC_LAUNCH("colstats", work, st, (k_colstats<uint16_t, true>), dim3(gx, gy), dim3(256), 0,
                  (const uint16_t*)W, n_out, n_in, ldw, part, rs);
    else
      WSIC_LAUNCH("colstats", work, st, (k_colstats<uint16_t, false>), dim3(gx, gy), dim3(256), 0,
                  (const uint16_t*)W, n_out, n_in, ldw, part, rs);
  } else {
    if (vec)
      WSIC_LAUNCH("colstats", work, st, (k_colstats<float, true>), dim3(gx, gy), dim3(256), 0,
                  (const float*)W, n_out, n_in, ldw, part, rs);
    else
      WSIC_LAUNCH("colstats", work, st, (k_colstats<float, false>), dim3(gx, gy), dim3(256), 0,
                  (const float*)W, n_out, n_in, ldw, part, rs);
  }
  WSIC_LAUNCH("colstats", 16.0 * gy * n_in, st, k_colstats_finish,
              dim3((unsigned)((n_in + 255) / 256)), dim3(256), 0, part, n_out, n_in, (int)gy, colvar);
  return WSIC_OK;
}

}  // namespace wsic
