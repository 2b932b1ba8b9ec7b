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
// its entries unconditionally (a zero leaves finished targets unchanged). Column j = 16a + r
// starts at 16 (a+1)(8a + r); a block holds 9216 doubles (72 KiB, two workgroups per CU).
#include "common.h"

namespace wsic {
namespace {

constexpr int BW = 128;                  // block width
constexpr int PACK = 9216;               // doubles per packed block
constexpr int pack_off(int j) { return 16 * ((j >> 4) + 1) * (8 * (j >> 4) + (j & 15)); }
static_assert(pack_off(BW) == PACK, "packed block size");

template <int L>
__device__ __forceinline__ double bcast_row(double v) {
  // row_newbcast:L -- lane L of each 16-lane DPP row to every lane of that row
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x150 + L, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x150 + L, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Step J of the in-block recursion (J = 127 ... 0), then the remaining ones. Columns past the
// end of a ragged last block hold z = 0 and all-zero B entries, so their steps change nothing
// and need no branch.
template <int J>
struct Steps {
  static __device__ __forceinline__ void run(double (&z)[8], const double* __restrict__ bl) {
    constexpr int a = J >> 4, l = J & 15, off = pack_off(J);
    const double qb = bcast_row<l>(rint(z[a]));
#pragma unroll
    for (int sp = 0; sp <= a; ++sp) z[sp] = fma(-bl[off + 16 * sp], qb, z[sp]);
    Steps<J - 1>::run(z, bl);
  }
};
template <>
struct Steps<-1> {
  static __device__ __forceinline__ void run(double (&)[8], const double*) {}
};

template <bool HAS_G, bool HAS_RESID>
__global__ __launch_bounds__(256) void k_sic_leaf(int64_t n_out, int64_t j0, int w,
                                                  const double* __restrict__ Y, int64_t ldy,
                                                  const double* __restrict__ G, int64_t ldg,
                                                  const double* __restrict__ Bpk,
                                                  const double* __restrict__ invd, double c,
                                                  double invc, int32_t* __restrict__ codes,
                                                  int64_t ldq, float* __restrict__ resid,
                                                  int64_t ldr, int* flags) {
  __shared__ __attribute__((aligned(16))) double Bs[PACK];
  const int tid = threadIdx.x;
  {
    // all 18 loads of a thread in flight before its LDS stores
    constexpr int PER = PACK / 2 / 256;
    static_assert(PER * 256 * 2 == PACK, "packed block is a whole number of 16-byte rounds");
    const uint4* src = reinterpret_cast<const uint4*>(Bpk);
    uint4* dst = reinterpret_cast<uint4*>(Bs);
    uint4 v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = src[e * 256 + tid];
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e * 256 + tid] = v[e];
  }

  const int l16 = tid & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool active = row < n_out;

  double z[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int j = l16 + 16 * s;
    double v = 0.0;
    if (active && j < w) {
      v = Y[row * ldy + j0 + j] * invc;
      if (HAS_G) v -= G[row * ldg + j0 + j];
    }
    z[s] = v;
  }
  __syncthreads();

  Steps<BW - 1>::run(z, Bs + l16);

  if (!active) return;
  int bad = 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int j = l16 + 16 * s;
    if (j < w) {
      const double q = rint(z[s]);
      int32_t qi = 0;
      if (q >= -2147483647.0 && q <= 2147483647.0) {
        qi = (int32_t)q;
      } else {
        bad |= (z[s] == z[s]) ? FLAG_RANGE : FLAG_NONFINITE;
      }
      codes[row * ldq + j0 + j] = qi;
      if (HAS_RESID) resid[row * ldr + j0 + j] = (float)((z[s] - q) * (c * invd[j0 + j]));
    }
  }
  if (bad) atomicOr(flags, bad);
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
  Bpk[blk * PACK + pack_off(j) + i] = v;
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

template <typename T>
__global__ void k_check_finite(const T* W, int64_t n_out, int64_t n_in, int64_t ldw, int* flags) {
  int bad = 0;
  const int64_t total = n_out * n_in;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / n_in, j = e % n_in;
    if (!isfinite(elem<T>(W, r * ldw + j))) bad = 1;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, FLAG_NONFINITE);
}

// Column sums of W and W^2 over a slab of COLSTAT_ROWS rows: 64 columns x 4 row lanes per
// workgroup, one partial pair per (slab, column); k_colstats_finish reduces the slabs in order.
constexpr int COLSTAT_ROWS = 256;
template <typename T>
__global__ __launch_bounds__(256) void k_colstats(const T* W, int64_t n_out, int64_t n_in,
                                                  int64_t ldw, double* part) {
  __shared__ double s1[4][64], s2[4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 + tx;
  const int64_t r0 = (int64_t)blockIdx.y * COLSTAT_ROWS;
  double a = 0.0, b = 0.0;
  if (j < n_in) {
    const int64_t r1 = (r0 + COLSTAT_ROWS < n_out) ? r0 + COLSTAT_ROWS : n_out;
    for (int64_t r = r0 + ty; r < r1; r += 4) {
      const double v = (double)elem<T>(W, r * ldw + j);
      a += v;
      b = fma(v, v, b);
    }
  }
  s1[ty][tx] = a;
  s2[ty][tx] = b;
  __syncthreads();
  if (ty == 0 && j < n_in) {
    const double sa = (s1[0][tx] + s1[1][tx]) + (s1[2][tx] + s1[3][tx]);
    const double sb = (s2[0][tx] + s2[1][tx]) + (s2[2][tx] + s2[3][tx]);
    part[((int64_t)blockIdx.y * n_in + j) * 2 + 0] = sa;
    part[((int64_t)blockIdx.y * n_in + j) * 2 + 1] = sb;
  }
}

__global__ void k_colstats_finish(const double* part, int64_t n_out, int64_t n_in, int nslab,
                                  double* colvar) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_in) return;
  double a = 0.0, b = 0.0;
  for (int s = 0; s < nslab; ++s) {
    a += part[((int64_t)s * n_in + j) * 2 + 0];
    b += part[((int64_t)s * n_in + j) * 2 + 1];
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

int launch_sic_leaf(int64_t n_out, int64_t j0, int w, const double* Y, int64_t ldy,
                    const double* G, int64_t ldg, const double* Bpk, const double* invd, double c,
                    int32_t* codes, int64_t ldq, float* resid, int64_t ldr, int* flags,
                    hipStream_t st) {
  if (w <= 0 || w > BW || j0 % BW != 0) {
    set_error("internal: leaf at %lld width %d", (long long)j0, w);
    return WSIC_E_INVAL;
  }
  const double* blk = Bpk + (j0 / BW) * PACK;
  const unsigned blocks = (unsigned)((n_out + 15) / 16);
  const double invc = 1.0 / c;
  // bytes that must stream: Y (+G) in, codes (+resid) out
  const double work = (double)n_out * w * (8.0 + (G ? 8.0 : 0.0) + 4.0 + (resid ? 4.0 : 0.0));
#define WSIC_LEAF(HG, HR)                                                                   \
  WSIC_LAUNCH("sic_leaf", work, st, (k_sic_leaf<HG, HR>), dim3(blocks), dim3(256), 0, n_out, \
              j0, w, Y, ldy, G, ldg, blk, invd, c, invc, codes, ldq, resid, ldr, flags)
  if (G) {
    if (resid)
      WSIC_LEAF(true, true);
    else
      WSIC_LEAF(true, false);
  } else {
    if (resid)
      WSIC_LEAF(false, true);
    else
      WSIC_LEAF(false, false);
  }
#undef WSIC_LEAF
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
  const int64_t total = n_out * n_in;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const double work = (double)total * (dtype == WSIC_BF16 ? 2.0 : 4.0);
  if (dtype == WSIC_BF16)
    WSIC_LAUNCH("check_finite", work, st, k_check_finite<uint16_t>, dim3((unsigned)blocks),
                dim3(256), 0, (const uint16_t*)W, n_out, n_in, ldw, flags);
  else
    WSIC_LAUNCH("check_finite", work, st, k_check_finite<float>, dim3((unsigned)blocks), dim3(256),
                0, (const float*)W, n_out, n_in, ldw, flags);
  return WSIC_OK;
}

int launch_colstats(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                    double* part, double* colvar, hipStream_t st) {
  const unsigned gx = (unsigned)((n_in + 63) / 64);
  const unsigned gy = (unsigned)((n_out + COLSTAT_ROWS - 1) / COLSTAT_ROWS);
  const double work = (double)n_out * n_in * (dtype == WSIC_BF16 ? 2.0 : 4.0);
  if (dtype == WSIC_BF16)
    WSIC_LAUNCH("colstats", work, st, k_colstats<uint16_t>, dim3(gx, gy), dim3(256), 0,
                (const uint16_t*)W, n_out, n_in, ldw, part);
  else
    WSIC_LAUNCH("colstats", work, st, k_colstats<float>, dim3(gx, gy), dim3(256), 0,
                (const float*)W, n_out, n_in, ldw, part);
  WSIC_LAUNCH("colstats", 16.0 * gy * n_in, st, k_colstats_finish,
              dim3((unsigned)((n_in + 255) / 256)), dim3(256), 0, part, n_out, n_in, (int)gy, colvar);
  return WSIC_OK;
}

}  // namespace wsic
