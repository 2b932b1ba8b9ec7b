// Internal declarations shared by the libwsic translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "wsic.h"

namespace wsic {

// ---------------------------------------------------------------- host-side error state
void set_error(const char* fmt, ...);
void clear_error();
const char* last_error();

#define WSIC_HIP_TRY(expr)                                                      \
  do {                                                                          \
    hipError_t _e = (expr);                                                     \
    if (_e != hipSuccess) {                                                     \
      ::wsic::set_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(_e),  \
                        __FILE__, __LINE__);                                    \
      return WSIC_E_HIP;                                                        \
    }                                                                           \
  } while (0)

// ---------------------------------------------------------------- launch timing
// While timing is on, a launch of a selected family carries a start and a stop event that the
// dispatch itself timestamps (hipExtLaunchKernelGGL), so the interval is the kernel's own
// execution, without marker packets around it.
struct ProfToken {
  int slot;
  hipEvent_t a, b;
};
ProfToken prof_begin(const char* family);
void prof_end(ProfToken t, double work);

#define WSIC_LAUNCH(family, work, stream, kernel, grid, block, shmem, ...)      \
  do {                                                                          \
    ::wsic::ProfToken _tok = ::wsic::prof_begin(family);                        \
    if (_tok.slot >= 0)                                                         \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, _tok.a, _tok.b, \
                            0, __VA_ARGS__);                                    \
    else                                                                        \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);      \
    ::wsic::prof_end(_tok, (double)(work));                                     \
    hipError_t _le = hipGetLastError();                                         \
    if (_le != hipSuccess) {                                                    \
      ::wsic::set_error("launch of %s failed: %s", #kernel,                     \
                        hipGetErrorString(_le));                                \
      return WSIC_E_HIP;                                                        \
    }                                                                           \
  } while (0)

// ---------------------------------------------------------------- device flags
// Small int array at the head of every workspace; kernels raise bits with atomicOr.
enum FlagBits : int {
  FLAG_NONFINITE = 1,
  FLAG_RANGE = 2,
  FLAG_BAD_DIAG = 4,
  FLAG_OVERFLOW_LIST = 8,
  FLAG_BAD_SCALE = 16,  // a class curvature that is not positive and finite
};

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- element access
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// ---------------------------------------------------------------- kernel launchers
// Each returns a wsic status; all work is enqueued on `st`.

// fp64 MFMA GEMM family: C[M x N] = beta*C + alpha * sum_k A'(m,k) B(n,k)
enum AMode : int {
  A_F64 = 0,      // A double, A'(m,k) = A[m*lda + k]
  A_F32 = 1,      // A float
  A_BF16 = 2,     // A bf16 bits
  A_CODES = 3,    // A int32 codes, A'(m,k) = vec[k] * A[m*lda + k]
  A_ERR_F32 = 4,  // A'(m,k) = W[m*lda+k] - vec[k] * Q[m*ldq+k], W float
  A_ERR_BF16 = 5, // same with W bf16
  A_F64_T = 6,    // A double stored k-major: A'(m,k) = A[k*lda + m]; B likewise B[k*ldb + n]
};
enum Epilogue : int { EPI_STORE = 0, EPI_SUMSQ = 1 };

struct GemmArgs {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  const int32_t* Q;
  int64_t ldq;
  const double* vec;
  const double* B;
  int64_t ldb;
  double* C;
  int64_t ldc;
  double alpha, beta;
  int tri;         // B(n,k) == 0 for k < n: each N-tile starts its K loop at its first column
  int upper_only;  // only tiles holding some n >= m are computed
  double* partial; // EPI_SUMSQ: one fp64 per tile
};
int gemm_tiles(const GemmArgs& g);  // number of tiles (size of `partial`)
// `work` = algorithmic flops of the call, recorded by the launch timer
int launch_gemm(int amode, int epi, const GemmArgs& g, const char* family, double work,
                hipStream_t st);

// Y = W U^T (setup of the SIC): W (dtype) M x K row-major, U fp64 with U[n][k] = 0 for k < n
// (the strict lower triangle is never read)
int launch_gemm_y(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                  const double* B, int64_t ldb, double* C, int64_t ldc, double work, hipStream_t st);

// covariance
// The tiles of the last, partial round of the covariance launch (the tile count is rarely a
// multiple of the CU count) are split along K into `pieces` workgroups each, which write their
// partial sums to a slot each in the workspace; a second launch adds them up. `full` tiles are
// computed whole.
constexpr int SPLIT_SLOTS = 256;     // workgroups the partial round is spread over
constexpr int SPLIT_MAX_PIECES = 16;
struct SyrkSplit {
  int64_t full;   // tiles computed whole
  int pieces;     // workgroups per split tile
  int64_t tail;   // split tiles
};
SyrkSplit syrk_split(int64_t n);
size_t syrk_split_bytes(int64_t n);  // workspace of the split (0: none)
int launch_syrk(const void* X, int dtype, int64_t rows, int64_t n, int64_t ldx, double alpha,
                double beta, double* S, int64_t lds, void* split_ws, size_t split_ws_bytes,
                hipStream_t st);
int launch_mirror_upper(double* S, int64_t n, int64_t lds, hipStream_t st);
int launch_diag_check(const double* S, int64_t n, int64_t lds, int* flags, hipStream_t st);

// cholesky
// factor the diagonal block at kb (into the 64 x 64 slot ud) and solve the block row to its
// right in place; launch_put_diag moves a slot's block into A
int launch_potrf_panel(double* A, int64_t lda, int64_t kb, int nbk, int64_t n, int64_t* info,
                       double* ud, hipStream_t st);
int launch_put_diag(double* A, int64_t lda, int64_t kb, int nbk, const double* ud, hipStream_t st);
int launch_zero_lower(double* A, int64_t n, int64_t lda, hipStream_t st);
// One 64-column step after the panel at kb: A[c0.., c0..] (upper tiles, c0 = kb + 64) -= X^T X
// with X the solved block row, fused with the panel at c0; chol_step_ok tells whether its
// alignment preconditions hold
bool chol_step_ok(const double* A, int64_t lda, int64_t c0);
int launch_chol_step(double* A, int64_t lda, int64_t kb, int64_t n, int64_t* info,
                     const double* ud_cur, double* ud_next, hipStream_t st);

// SIC
int launch_prep(const double* U, int64_t ldu, int64_t n, double* invd, int* flags, hipStream_t st);
// delta_j = c / U_jj (nullable), diag_j = U_jj (nullable)
int launch_delta(const double* U, int64_t ldu, int64_t n, double c, double* delta, double* diag,
                 hipStream_t st);
int launch_check_finite(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                        int* flags, hipStream_t st);
// packed diagonal blocks of B = U diag(1/U_jj) (c-independent), consumed by the leaf
int sic_pack_doubles(int64_t n_in);
int launch_pack_blocks(const double* U, int64_t ldu, int64_t n, const double* invd, double* Bpk,
                       hipStream_t st);
// Integer form of the interference product: NL int8 digits per B entry (P = 8 NL - 2 bits
// of fixed point per row), codes clamped to +-127 with the excess of larger codes kept in a
// per-row list of OCAP entries.
constexpr int LIMBS = 5;
constexpr double LIMB_EPS = 1.0 / (double)(1ull << (8 * LIMBS - 2));  // 2^-P
constexpr int OCAP = 64;
// rows per workgroup of the residual distortion pass (its partials are sized from it)
constexpr int DIST_ROWS = 32;

struct LeafArgs {
  int64_t n_out, n_in, j0;
  int w;
  const double* Y;
  int64_t ldy;
  const double* G;  // null for the rightmost block
  int64_t ldg;
  const double* Bpk;
  const double* invd;
  double c, invc;
  int32_t* codes;
  int64_t ldq;
  float* resid;  // nullable
  int64_t ldr;
  int* flags;
  // integer interference mode
  const double* U;
  int64_t ldu;
  const double* bscale;  // 2^e_j
  double guard_scale;    // multiplies the error bound (1 in normal use)
  int8_t* q8;
  int64_t ldq8;
  double* absq;  // per row: sum |q| over the columns done so far in this pass
  int* ocnt;     // per row: entries in the excess list
  int2* olist;   // per row: OCAP (column, q - clamp(q)) pairs
  // interference of the finished columns [kf0, kf0 + kf) formed inside the leaf from the int8
  // digit planes (kf = 0: none)
  const int8_t* D;        // digit plane 0 (row j, column k at D[j * ldd + k])
  int64_t ldd, plane;
  const double* escale;   // 2^(e_j - P)
  int64_t kf0;
  int kf;
  int w_bytes;  // bytes per weight of the layer (2 bf16, 4 f32): the algorithmic byte count
};
int launch_sic_leaf(const LeafArgs& p, bool i8, hipStream_t st);
// int8 mode: up to 4 blocks [j0, j0 + w) in one launch (w <= 512), interference of the range's
// finished columns formed inside; G (nullable) holds the interference of the columns >= j0 + w
int launch_sic_super(const LeafArgs& p, hipStream_t st);

int launch_limb_pack(const double* U, int64_t ldu, int64_t n, const double* invd, double* escale,
                     double* bscale, int8_t* D, int64_t ldd, hipStream_t st);
int launch_gemm_i8(int64_t M, int64_t N, int64_t K, const int8_t* A8, int64_t lda, const int8_t* D,
                   int64_t ldd, int64_t plane, const double* escale, double* C, int64_t ldc,
                   double beta, hipStream_t st);
int colstats_doubles(int64_t n_out, int64_t n_in);
// column variances of diag(rs) W (rs nullable: W itself); part (colstats_doubles, 16-byte aligned)
int launch_colstats(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                    double* part, double* colvar, hipStream_t st, const double* rs = nullptr);

// histogram / entropy
constexpr int HIST_HALF = 2047;
constexpr int HIST_BINS = 2 * HIST_HALF + 1;
constexpr unsigned OVF_CAP = 1u << 20;
struct EntropyResult {
  double sum_nlogn;            // sum over window bins of n log2 n
  unsigned long long nsym;     // non-empty window bins
  unsigned int ovf_count;      // codes outside the window
  int flags;                   // flags word of the pass (when given)
  int aux;                     // its second word: workgroups re-derived in fp64
  int aux2;                    // its third word: decisions re-checked one by one
};
int launch_hist(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                unsigned long long* bins, int32_t* ovf, unsigned int* ovf_count, hipStream_t st);
int launch_entropy_reduce(const unsigned long long* bins, const unsigned int* ovf_count,
                          const int* flags, EntropyResult* res, hipStream_t st);
int launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// distortion
int launch_dist_resid(const float* resid, int64_t n_out, int64_t n_in, int64_t ldr,
                      const double* U, int64_t ldu, double* partial, int nblk, hipStream_t st);
// W_hat_ij = c q_ij / (U_jj rs_i) (rs nullable: 1)
int launch_dequant(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                   const double* invd, double c, void* W_hat, int w_hat_dtype, int64_t ldh,
                   hipStream_t st, const double* rs = nullptr);

// per-column histograms: 32 columns x 512 rows per workgroup, LDS window +-127 per column
constexpr int COL_TILE = 32, COL_ROWS = 512, COL_HALF = 127, COL_BINS = 2 * COL_HALF + 1;
int launch_hist_cols(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                     unsigned* colbins, int2* ovf, unsigned* ovf_count, hipStream_t st);
int launch_col_entropy(const unsigned* colbins, int64_t n_in, double* colS, hipStream_t st);
// partial sums of W^2 over nblk workgroups; log2 U_jj per column (FLAG_BAD_DIAG if not positive)
int launch_sumsq(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw, double* partial,
                 int nblk, hipStream_t st);
int launch_logdiag(const double* U, int64_t ldu, int64_t n, double* out, int* flags, hipStream_t st);

// LMMSE row factors from Y = W U^T and the SIC residuals; dead-feature removal
int launch_lmmse_rows(const double* Y, int64_t ldy, const float* R, int64_t ldr, const double* U,
                      int64_t ldu, int64_t n_out, int64_t n_in, double* gamma, double* dbefore,
                      double* dafter, hipStream_t st);
int launch_live_scan(const double* S, int64_t n, int64_t lds, double tau, int32_t* idx,
                     int32_t* pos, long long* live_count, int* flags, hipStream_t st);
int launch_gather_features(const void* W, int dtype, int64_t n_out, int64_t ldw, const double* S,
                           int64_t lds, const int32_t* idx, int64_t n_live, void* Wl, int64_t ldwl,
                           double* Sl, int64_t ldsl, hipStream_t st);
int launch_scatter_codes(const int32_t* ql, int64_t ldql, const int32_t* pos, int64_t n_in,
                         int64_t n_out, int32_t* q, int64_t ldq, hipStream_t st);

// rANS coder of the codes
int launch_rans_esc_count(const int32_t* q, int64_t N, int L, int64_t G, uint32_t* cnt, hipStream_t st);
int launch_scan_u32(const uint32_t* in, int64_t n, uint32_t* out, hipStream_t st);
int launch_rans_encode(const int32_t* q, int64_t N, int L, int64_t G, int lo, int nsym,
                       const uint16_t* freq, const uint32_t* eofs, int32_t* esc_out, uint16_t* temp,
                       uint32_t* gwords, uint32_t* states, hipStream_t st);
int launch_rans_compact(const uint16_t* temp, int L, int64_t G, const uint32_t* gwords,
                        const uint32_t* gofs, uint16_t* payload, hipStream_t st);
int launch_rans_decode(int mode, const uint16_t* freq, int nsym, int lo, int64_t N, int L, int64_t G,
                       const uint32_t* gofs, const uint32_t* eofs, const uint32_t* states,
                       const int32_t* escapes, uint32_t n_esc, const uint16_t* payload,
                       uint32_t n_words, void* out, int64_t n_in, const double* invd, double c,
                       int* flags, hipStream_t st);

// softmax curvature (SoftWater): logits, row normalizers, per-class sums
struct CurvArgs {
  const void* X;
  const void* W;
  int dtype;
  int64_t rows, n, ldx, K, ldw;
  double eps, alpha, beta;
  double* lam;       // K, in/out
  int* flags;
  float* Lg;         // rows x ldl logits
  int64_t ldl;
  float2* part;      // rows x ntn (max, sum exp) per class tile
  float* rmax;       // rows
  double* rinvz;     // rows
  double* cpart;     // nchunk x K
  bool force_generic;
};
void curvature_dims(int64_t rows, int64_t K, int64_t* ntn, int64_t* nchunk, int64_t* ldl);
int launch_softmax_curvature(const CurvArgs& a, hipStream_t st);
// s_k = sqrt(lam_k) (FLAG_BAD_SCALE unless lam_k is positive and finite)
int launch_row_sqrt(const double* lam, int64_t n, double* s, int* flags, hipStream_t st);
// Y[r, :] *= s[r]
int launch_scale_rows(double* Y, int64_t n_out, int64_t n_in, int64_t ldy, const double* s,
                      hipStream_t st);
// the rate controller's probe layer: K groups of S evenly spaced rows of Y, group g scaled by
// fac.v[g] (S * K <= 65535, S <= n_out, K <= PROBE_MAX)
constexpr int PROBE_MAX = 8;
struct ProbeFactors {
  double v[PROBE_MAX];
};
int launch_probe_rows(const double* Y, int64_t ldy, int64_t n_out, int64_t n_in, int S, int K,
                      const ProbeFactors& fac, double* Yp, int64_t ldp, hipStream_t st);
int launch_sum_partials(const double* partial, int64_t n, double* out, hipStream_t st);

}  // namespace wsic
