/*
 * wsic.h -- C ABI of libwsic: WaterSIC quantization of one linear layer on an MI355X (gfx950).
 *
 * Method (web page "WaterSIC: information-theoretically (near) optimal linear layer
 * quantization", gist.science; sections cited as [WaterSIC <section>]):
 *   Sigma = X^T X / N                         calibration covariance  [Sommario tecnico §2 item 1]
 *   Sigma = U^T U, U upper, U_jj > 0           Cholesky (the page's L L^T with U = L^T) [§2 item 1]
 *   Delta_j = c / U_jj                         waterfilling steps, alpha_i ~ 1/|l_ii| [§2 item 2]
 *   SIC, columns j = n_in-1 ... 0:             interference cancellation in reverse order [§2 item 1]
 *       t_j = w_j + sum_{k>j} (U_jk/U_jj) (w_k - Delta_k q_k),  q_j = rint(t_j / Delta_j)
 *   rate = empirical entropy of the pooled codes (unbounded integers, entropy coded) [§2 item 3]
 *   distortion = tr((W - W_hat) Sigma (W - W_hat)^T)  (output error of Y = W X) [§1]
 *
 * Conventions for every call:
 *   - Return value: WSIC_OK (0) or a negative WSIC_E_* status. Nothing is thrown across the ABI.
 *     wsic_last_error() gives a message for the last failing call on the calling thread.
 *   - Array arguments are DEVICE pointers owned by the caller, row-major, with explicit
 *     leading dimensions in elements (ld >= number of columns). Host pointers are marked
 *     "host". Inputs are const and never written.
 *   - Scratch memory is the caller's: query wsic_workspace_bytes(op, n_out, n_in) and pass
 *     ws / ws_bytes. A smaller ws_bytes returns WSIC_E_WORKSPACE. The library allocates no
 *     device memory of its own.
 *   - stream is a hipStream_t (NULL = legacy default stream). All device work is enqueued on
 *     it. Calls that return host scalars synchronize that stream before returning.
 *   - dtype selects the element type of W / X: WSIC_F32 (float) or WSIC_BF16 (bfloat16 bits).
 *   - Sigma and U are fp64 n_in x n_in.
 *   - Calls are re-entrant only on distinct workspaces.
 */
#ifndef WSIC_H
#define WSIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WSIC_VERSION 100

enum wsic_status {
  WSIC_OK = 0,
  WSIC_E_INVAL = -1,       /* bad argument: null pointer, size <= 0, ld too small, bad enum */
  WSIC_E_NOT_PD = -2,      /* covariance not positive definite (see info) */
  WSIC_E_NONFINITE = -3,   /* NaN / Inf in an input */
  WSIC_E_NO_BRACKET = -4,  /* target rate not reachable by any grid scale */
  WSIC_E_RANGE = -5,       /* a code does not fit int32, or too many distinct large codes */
  WSIC_E_WORKSPACE = -6,   /* ws_bytes smaller than wsic_workspace_bytes() */
  WSIC_E_HIP = -7          /* a HIP runtime call failed */
};

enum wsic_dtype { WSIC_F32 = 0, WSIC_BF16 = 1 };

enum wsic_op {
  WSIC_OP_COVARIANCE = 0,
  WSIC_OP_CHOLESKY = 1,
  WSIC_OP_SIC = 2,
  WSIC_OP_WATERFILL = 3,
  WSIC_OP_ENTROPY = 4,
  WSIC_OP_DISTORTION = 5,
  WSIC_OP_CURVATURE = 6,       /* n_out = calibration rows of one call, n_in = classes K */
  WSIC_OP_SOFTWATER = 7,       /* wsic_softwater_waterfill on an n_out x n_in layer       */
  WSIC_OP_SOFTWATER_DIST = 8,  /* wsic_softwater_distortion                               */
  WSIC_OP_ENTROPY_COLUMNS = 9, /* wsic_entropy_columns on an n_out x n_in code matrix      */
  WSIC_OP_GAUSS_RATE = 10,     /* wsic_gaussian_rate                                      */
  WSIC_OP_LMMSE = 11,          /* wsic_lmmse_scale                                        */
  WSIC_OP_LIVE = 12,           /* wsic_live_features (n_in = size of Sigma)               */
  WSIC_OP_RANS_ENC = 13,       /* wsic_rans_encode: n_out = lane_symbols, n_in = codes    */
  WSIC_OP_RANS_DEC = 14        /* wsic_rans_decode(_dequant): n_in = layer columns (1)    */
};

enum wsic_dmode { WSIC_D_RESID = 0, WSIC_D_DIRECT = 1 };
enum wsic_wfmode { WSIC_WF_AUTO = 0, WSIC_WF_SECANT = 1, WSIC_WF_BISECT = 2 };
/* What the rate controller holds to the target: the entropy of all codes pooled into one table,
 * or the mean over input columns of each column's code entropy (one entropy code per column,
 * the setting of the rate gap in [WaterSIC §3]). */
enum wsic_ratemode { WSIC_RATE_POOLED = 0, WSIC_RATE_COLUMNS = 1 };

/* WSIC_WF_AUTO picks BISECT for layers of fewer than WSIC_WF_AUTO_PARAMS weights, SECANT
 * otherwise. */
#define WSIC_WF_AUTO_PARAMS (1LL << 20)

/* Library version (WSIC_VERSION). */
int wsic_version(void);

/* Message for the last failing call on this thread ("" if none). Owned by the library. */
const char* wsic_last_error(void);

/* Static name of a status code. */
const char* wsic_status_str(int status);

/* Bytes of device workspace that call `op` needs for an n_out x n_in layer (n_out is ignored
 * by WSIC_OP_COVARIANCE / WSIC_OP_CHOLESKY / WSIC_OP_LIVE; for WSIC_OP_ENTROPY pass the code
 * matrix shape).
 * Returns 0 for an unknown op. */
size_t wsic_workspace_bytes(int op, int64_t n_out, int64_t n_in);

/*
 * Calibration covariance [WaterSIC §2 item 1], SYRK semantics:
 *     Sigma <- beta * Sigma + alpha * X^T X
 * X: rows x n_in, ldx >= n_in, dtype f32 or bf16. Sigma: n_in x n_in fp64, lds >= n_in.
 * To accumulate Sigma = X^T X / N over streamed chunks, pass alpha = 1/N for every chunk,
 * beta = 0 for the first chunk and beta = 1 afterwards. Only the upper triangle of the old
 * Sigma is read; the full symmetric result is written. bf16 chunks run on bf16 MFMA with
 * fp32 partial sums over at most 64 rows folded into fp64; f32 chunks run in fp64.
 * Errors: WSIC_E_INVAL; WSIC_E_NONFINITE if X holds NaN/Inf (Sigma is then unspecified).
 */
int wsic_covariance(const void* X, int dtype, int64_t rows, int64_t n_in, int64_t ldx,
                    double alpha, double beta, double* Sigma, int64_t lds,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * Cholesky factorization in place [WaterSIC §2 item 1]: on return the upper triangle of A
 * holds U with Sigma = U^T U and U_jj > 0, and the strict lower triangle is zero.
 * A: n x n fp64, lda >= n. Only the upper triangle of the input is read.
 * *info (host): 0 on success, else the 1-based index of the first pivot that is not positive
 * (or not finite); the call then returns WSIC_E_NOT_PD and A is unspecified.
 */
int wsic_cholesky(double* A, int64_t n, int64_t lda, int64_t* info,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * One SIC pass at grid scale c [WaterSIC §2 items 1-2]: steps Delta_j = c / U_jj, columns
 * visited j = n_in-1 ... 0, each rounded (ties to even) after cancelling the interference of
 * the columns already quantized. Computed in fp64.
 * W: n_out x n_in (dtype), ldw >= n_in. U: upper factor from wsic_cholesky, ldu >= n_in; its
 * strict lower triangle is never read (here and in wsic_waterfill / wsic_distortion).
 * codes (out): n_out x n_in int32, ldq >= n_in.
 * resid (out, nullable): n_out x n_in float, ldr >= n_in, r_j = t_j - Delta_j q_j in the
 * units of W (|r_j| <= Delta_j / 2); sum_j U_jj^2 ||r_:,j||^2 is the layer distortion.
 * Errors: WSIC_E_INVAL (c <= 0 or not finite), WSIC_E_NONFINITE (W), WSIC_E_RANGE (a code
 * outside int32).
 */
int wsic_sic_quantize(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                      const double* U, int64_t ldu, double c,
                      int32_t* codes, int64_t ldq, float* resid, int64_t ldr,
                      void* ws, size_t ws_bytes, void* stream);

/* Default acceptance window of the rate controller (bits per weight). The pooled entropy of SIC
 * codes is not smooth below ~1e-4 relative changes of c (one flipped rounding decision re-routes
 * the interference of every column left of it, moving H by a few 1e-5), so a window narrower
 * than that costs extra passes. */
#define WSIC_WF_RATE_TOL 8e-5

/* Options of the rate controller; pass NULL for the defaults shown. */
typedef struct wsic_wf_opts {
  double rate_tol;     /* accept c once R - rate_tol < H(c) <= R (default WSIC_WF_RATE_TOL)  */
  double bracket_log2; /* or once log2(c_hi / c_lo) <= bracket_log2 (default 2^-20)          */
  int32_t max_passes;  /* SIC passes allowed (default 64)                                   */
  int32_t mode;        /* WSIC_WF_BISECT: start at c_init, double (halve) c until the rate
                          is bracketed, then geometric bisection, stopping only on
                          bracket_log2 -- the reference search, whose sequence of grid
                          scales is fully determined by the code entropies it sees;
                          WSIC_WF_SECANT: safeguarded regula falsi (Illinois) on log2 c,
                          far fewer passes once H(c) is smooth (large layers); on layers
                          of at least 16384 rows its first pass is a probe of 8 grid scales
                          on 512 evenly spaced rows (counted in passes_out), which gives the
                          start and the slope;
                          WSIC_WF_AUTO (default): BISECT below WSIC_WF_AUTO_PARAMS weights,
                          where H(c) moves in visible non-monotone steps, else SECANT     */
  double c_init;       /* > 0: first grid scale tried; 0: high-rate estimate
                          sqrt(2 pi e mean_j(var(W_:,j) U_jj^2)) 2^-R                        */
  int32_t rate_mode;   /* WSIC_RATE_POOLED (default) or WSIC_RATE_COLUMNS                    */
  int32_t reserved;    /* 0                                                                  */
} wsic_wf_opts;

/*
 * Waterfilling rate allocation [WaterSIC §2 items 2-3]: finds the grid scale c (the smallest,
 * to the controller's tolerance) whose SIC codes have pooled empirical entropy
 * H(c) <= target_bits, and returns those codes.
 * Outputs (host): *c_out, *rate_out = H(c) in bits per weight, *passes_out = SIC passes run.
 * codes (out, required) / resid (out, nullable): as in wsic_sic_quantize, at c_out.
 * Errors: as wsic_sic_quantize, WSIC_E_INVAL for target_bits <= 0, WSIC_E_NO_BRACKET when
 * the target cannot be met within max_passes / 64 doublings.
 */
int wsic_waterfill(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                   const double* U, int64_t ldu, double target_bits, const wsic_wf_opts* opts,
                   double* c_out, double* rate_out, int32_t* passes_out,
                   int32_t* codes, int64_t ldq, float* resid, int64_t ldr,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Zeroth-order empirical entropy of the pooled codes [WaterSIC §2 item 3]:
 *   H = log2(N) - (1/N) sum_k n_k log2 n_k   bits per code, N = n_out * n_in.
 * codes: n_out x n_in int32, ldq >= n_in. *bits_per_param (host). *n_symbols (host,
 * nullable): number of distinct codes. Codes beyond +-2047 are counted through an overflow
 * list of bounded size (WSIC_E_RANGE if more than 2^20 such codes).
 */
int wsic_entropy(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                 double* bits_per_param, int64_t* n_symbols,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Mean per-column code entropy [WaterSIC §3, §2 item 3]:
 *   H = (1/n_in) sum_j H(codes[:, j]) = log2(n_out) - (1/N) sum_j sum_k n_jk log2 n_jk,
 * N = n_out * n_in, in bits per code. It never exceeds the pooled entropy (wsic_entropy).
 * codes: n_out x n_in int32, ldq >= n_in; *bits_per_param (host). Codes beyond +-127 are counted
 * through an overflow list of bounded size (WSIC_E_RANGE if more than 2^20 such codes).
 * Workspace: wsic_workspace_bytes(WSIC_OP_ENTROPY_COLUMNS, n_out, n_in).
 */
int wsic_entropy_columns(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                         double* bits_per_param, void* ws, size_t ws_bytes, void* stream);

/*
 * Gaussian rate-distortion limit of a layer at distortion D [WaterSIC §3 Limiti teorici: the
 * limit is a reverse waterfilling; WaterSIC is within 1/2 log2(2 pi e / 12) = 0.2546 bit of it
 * at high rate]. Rows of W are modelled as N(0, var I) with var = mean of W^2 (*var_out, host,
 * nullable); the distortion per weight theta = D / (n_out n_in) is taken below every eigenvalue
 * of var * Sigma (the high-rate regime), where the limit is
 *   *rate_out (host) = 1/2 log2(var / theta) + (1/n_in) sum_j log2 U_jj   bits per weight
 * (det Sigma = prod U_jj^2). When theta exceeds the smallest eigenvalue of var * Sigma this
 * form is below the true limit (reverse waterfilling raises it); the caller owns that check.
 * Workspace: wsic_workspace_bytes(WSIC_OP_GAUSS_RATE, n_out, n_in).
 */
int wsic_gaussian_rate(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                       const double* U, int64_t ldu, double D, double* rate_out, double* var_out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * LMMSE rescale [WaterSIC §2 item 4, "Correzione LMMSE": a linear factor that corrects the
 * bias of rounding], one factor per output row:
 *   gamma_k = (w_k Sigma w_hat_k^T) / (w_hat_k Sigma w_hat_k^T)
 * minimizes the row's output error (w_k - gamma w_hat_k) Sigma (w_k - gamma w_hat_k)^T; the
 * rescaled row is gamma_k w_hat_k. Computed from Y = W U^T and the SIC residuals (resid from
 * wsic_sic_quantize / wsic_waterfill, required): U w_hat_k^T = U w_k^T - diag(U) r_k.
 * gamma (out): n_out fp64 (device); a row quantized to zero keeps gamma = 1.
 * *D_before, *D_after (host, nullable): tr(E Sigma E^T) without and with the factors.
 * Workspace: wsic_workspace_bytes(WSIC_OP_LMMSE, n_out, n_in).
 */
int wsic_lmmse_scale(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                     const double* U, int64_t ldu, const float* resid, int64_t ldr, double* gamma,
                     double* D_before, double* D_after, void* ws, size_t ws_bytes, void* stream);

/*
 * Dead-feature removal [WaterSIC §2 item 4, "Cancellazione delle Feature Morte": input
 * dimensions of near-zero variance are removed so that the Cholesky factorization stays stable].
 * A column i is live when Sigma_ii > tau * max_j Sigma_jj (0 <= tau < 1).
 * wsic_live_features: idx (out, device, n): the live columns in ascending order, idx[0, *n_live);
 *   pos (out, device, n): each column's position in idx, -1 for a dead one; *n_live (host).
 *   WSIC_E_INVAL when no column is live. Workspace: wsic_workspace_bytes(WSIC_OP_LIVE, 0, n).
 * wsic_gather_features: W_live = W[:, idx] (n_out x n_live, same dtype, ldwl >= n_live) and, if
 *   Sigma is given, Sigma_live = Sigma[idx][:, idx] (n_live x n_live, ldsl >= n_live). The
 *   quantization then runs on the live layer (wsic_cholesky, wsic_waterfill, ...).
 * wsic_scatter_codes: codes[:, j] = codes_live[:, pos[j]] for live j, 0 for dead j (a dead
 *   column's weights multiply inputs of no variance: they are dropped).
 */
int wsic_live_features(const double* Sigma, int64_t n, int64_t lds, double tau, int32_t* idx,
                       int32_t* pos, int64_t* n_live, void* ws, size_t ws_bytes, void* stream);
int wsic_gather_features(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                         const double* Sigma, int64_t lds, const int32_t* idx, int64_t n_live,
                         void* W_live, int64_t ldwl, double* Sigma_live, int64_t ldsl,
                         void* stream);
int wsic_scatter_codes(const int32_t* codes_live, int64_t n_out, int64_t ldql, const int32_t* pos,
                       int64_t n_in, int32_t* codes, int64_t ldq, void* stream);

/*
 * Entropy coder of the codes [WaterSIC §2 item 3: the integer codes are stored without a fixed
 * range through an entropy coder; the rate of the layer is the coder's output]. rANS with a static
 * table (the pooled histogram of the codes within +-2047 scaled to 2^14, plus an escape symbol for
 * wider codes, stored raw), 32-bit states, 16-bit words; 64 interleaved streams per group, lane l
 * of group g coding the codes (g L + k) 64 + l, k < L (L = lane_symbols), with the group's words
 * in decoding order. The container (device memory, little endian) holds a 64-byte header, the
 * table, per-group word and escape offsets, the streams' initial states, the escapes and the
 * 16-bit payload.
 * wsic_rans_bound: container bytes that suffice for n codes.
 * wsic_rans_encode: codes n contiguous int32 (flattened row-major); out: device buffer of
 *   out_cap >= wsic_rans_bound(n, L) bytes; *out_bytes (host): bytes written. n < 2^31.
 *   Workspace: wsic_workspace_bytes(WSIC_OP_RANS_ENC, lane_symbols, n).
 * wsic_rans_decode: the n codes back (n must match the container); WSIC_E_INVAL for a container
 *   that is not one, whose frequency table does not sum to 2^14, whose streams read past the
 *   escapes or the payload, or that does not decode to the encoder's start states (a damaged
 *   container never makes the decoder read or write outside its buffers).
 *   Workspace: wsic_workspace_bytes(WSIC_OP_RANS_DEC, 0, 1).
 * wsic_rans_decode_dequant: decodes an n_out x n_in layer straight to W_hat_ij = c q_ij / U_jj
 *   (w_hat_dtype f32 or bf16, contiguous). Workspace: wsic_workspace_bytes(WSIC_OP_RANS_DEC, 0, n_in).
 */
size_t wsic_rans_bound(int64_t n, int32_t lane_symbols);
int wsic_rans_encode(const int32_t* codes, int64_t n, int32_t lane_symbols, uint8_t* out,
                     size_t out_cap, size_t* out_bytes, void* ws, size_t ws_bytes, void* stream);
int wsic_rans_decode(const uint8_t* in, size_t in_bytes, int32_t* codes, int64_t n, void* ws,
                     size_t ws_bytes, void* stream);
int wsic_rans_decode_dequant(const uint8_t* in, size_t in_bytes, int64_t n_out, int64_t n_in,
                             const double* U, int64_t ldu, double c, void* W_hat, int w_hat_dtype,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Layer distortion [WaterSIC §1]: D = tr((W - W_hat) Sigma (W - W_hat)^T), W_hat_ij = Delta_j q_ij.
 *   mode WSIC_D_RESID : D = sum_j U_jj^2 sum_i r_ij^2 from the SIC residuals (resid required);
 *                       a streaming pass.
 *   mode WSIC_D_DIRECT: D = ||(W - W_hat) U^T||_F^2 by an fp64 MFMA product (resid ignored).
 * W_hat (out, nullable): n_out x n_in of dtype w_hat_dtype, ldh >= n_in.
 * *D_out (host).
 */
int wsic_distortion(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                    const int32_t* codes, int64_t ldq, const double* U, int64_t ldu, double c,
                    const float* resid, int64_t ldr, int mode, double* D_out,
                    void* W_hat, int w_hat_dtype, int64_t ldh,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------------------------
 * SoftWater: class-aware rate allocation for a softmax output layer (web page "SoftWater:
 * Class-Aware Rate Allocation for Softmax Quantization", Portuguese technical summary, §2).
 * The layer W (K classes x n inputs, logits W x) is quantized by SIC on the grids
 *     Delta_kj = c / (sqrt(lambda_k) U_jj),   lambda_k = E[p~_k (1 - p~_k)],
 * [SoftWater §2 "Aproximação Tratável"], p = softmax(W x) over the calibration inputs, mixed
 * with the uniform distribution: p~ = (1 - smoothing) p + smoothing / K [§2 "Prior de
 * Suavização"]. The distortion is the second-order KL estimate
 *     D = 1/2 sum_k lambda_k (w_k - w_hat_k) Sigma (w_k - w_hat_k)^T   [§2 "Derivação do Objetivo"].
 * ---------------------------------------------------------------------------------------------
 */

/*
 * Class curvatures from one chunk of calibration inputs, accumulated like wsic_covariance:
 *     lambda <- beta * lambda + alpha * sum_{rows x} p~(x) (1 - p~(x))     (elementwise, K)
 * Pass alpha = 1/N_total for every chunk, beta = 0 for the first and 1 afterwards.
 * X: rows x n_in, ldx >= n_in; W: n_classes x n_in, ldw >= n_in; both of `dtype`.
 * lambda: n_classes fp64 (device). smoothing in [0, 1].
 * bf16 inputs with n_in, ldx, ldw multiples of 8 (16-byte aligned) run the logits on bf16 MFMA
 * with fp32 sums; other shapes and f32 inputs sum in fp64. The logits of the chunk are kept in
 * the workspace (rows x K fp32): split large calibration sets into chunks of rows.
 * Workspace: wsic_workspace_bytes(WSIC_OP_CURVATURE, rows, n_classes).
 * Errors: WSIC_E_INVAL; WSIC_E_NONFINITE (X or W holds NaN/Inf, or the result is not finite).
 */
int wsic_softmax_curvature(const void* X, int dtype, int64_t rows, int64_t n_in, int64_t ldx,
                           const void* W, int64_t n_classes, int64_t ldw, double smoothing,
                           double alpha, double beta, double* lambda, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Waterfilling with the class-aware grids [SoftWater §2 "Implementação": SIC as in WaterSIC,
 * rows rescaled per class]: as wsic_waterfill, with row k's steps divided by sqrt(lambda[k]).
 * lambda: n_out fp64 (device), every entry positive and finite (else WSIC_E_INVAL).
 * resid (nullable) holds the residuals of the rescaled rows, sqrt(lambda_k) (t_kj - Delta_kj
 * q_kj), so that sum_j U_jj^2 sum_k resid_kj^2 = 2 D.
 * Workspace: wsic_workspace_bytes(WSIC_OP_SOFTWATER, n_out, n_in).
 */
int wsic_softwater_waterfill(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                             const double* U, int64_t ldu, const double* lambda,
                             double target_bits, const wsic_wf_opts* opts, double* c_out,
                             double* rate_out, int32_t* passes_out, int32_t* codes, int64_t ldq,
                             float* resid, int64_t ldr, void* ws, size_t ws_bytes, void* stream);

/*
 * KL distortion estimate of a SoftWater quantization [SoftWater §2 "Derivação do Objetivo"]:
 * *D_out (host) = 1/2 sum_j U_jj^2 sum_k resid_kj^2 from the residuals returned by
 * wsic_softwater_waterfill (resid required). W_hat (out, nullable): c q_kj / (sqrt(lambda_k)
 * U_jj) as w_hat_dtype, ldh >= n_in.
 * Workspace: wsic_workspace_bytes(WSIC_OP_SOFTWATER_DIST, n_out, n_in).
 */
int wsic_softwater_distortion(const int32_t* codes, int64_t n_out, int64_t n_in, int64_t ldq,
                              const double* U, int64_t ldu, double c, const double* lambda,
                              const float* resid, int64_t ldr, double* D_out, void* W_hat,
                              int w_hat_dtype, int64_t ldh, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * Layer distortion with no allocation of any kind, for callers that cannot allocate device or
 * pinned host memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments and results as wsic_distortion, without the workspace: the scratch
 * is a static device buffer of WSIC_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends,
 * and *D_out is read back by a plain copy into the caller's host memory.
 * The device is the one current on the calling thread; stream must belong to it.
 * Returns WSIC_E_WORKSPACE when the layer needs more scratch than the buffer holds
 * (wsic_workspace_bytes(WSIC_OP_DISTORTION, n_out, n_in) > WSIC_NOALLOC_SCRATCH_BYTES, about
 * 16 n_in + 8 max(ceil(n_out / 64) ceil(n_in / 64), ceil(n_out / 32) ceil(n_in / 1024)) bytes;
 * 8192 x 28672 and 32000 x 4096 fit).
 * All calls on one GPU share its buffer: calls that overlap in time on one GPU (different
 * streams or threads) race and give undefined results; run them one after another.
 */
#define WSIC_NOALLOC_SCRATCH_BYTES (1u << 20)
int wsic_distortion_noalloc(const void* W, int dtype, int64_t n_out, int64_t n_in, int64_t ldw,
                            const int32_t* codes, int64_t ldq, const double* U, int64_t ldu,
                            double c, const float* resid, int64_t ldr, int mode, double* D_out,
                            void* W_hat, int w_hat_dtype, int64_t ldh, void* stream);

/*
 * Diagnostic switches (process-wide, default off). They select alternative kernel paths that
 * compute the same results, so that tests can compare the paths with each other and with the
 * reference; nothing in normal use needs them. Set them only while no other library call runs.
 *   WSIC_DBG_FP64_PRODUCT   1: the SIC interference by the fp64 MFMA product instead of the
 *                              exact int8 digit-plane product (default 0)
 *   WSIC_DBG_SUPER_BLOCKS   0: one SIC launch per 128-column block instead of up to four
 *                              (default 1)
 *   WSIC_DBG_GUARD_SCALE    >= 1: multiplies the int8 product's error bound, so that more
 *                              rounding decisions are re-checked in fp64 (default 1); values
 *                              below 1 are refused (they would weaken the exactness guarantee)
 *   WSIC_DBG_CHOL_FUSED     0: Cholesky update and next panel as separate launches (default 1)
 *   WSIC_DBG_LOGITS_GENERIC 1: fp64 VALU logits for bf16 curvature inputs too (default 0)
 *   WSIC_DBG_TRACE          1: one line per SIC pass of the rate controller on stderr (default 0)
 *   WSIC_DBG_PROBE          0: the secant controller starts from its rate model alone, without
 *                              the probe pass (8 grid scales on 512 sampled rows, layers of at
 *                              least 16384 rows; default 1); the accepted c then differs within
 *                              the controller's tolerance
 * wsic_debug_set returns WSIC_E_INVAL for an unknown knob or a value out of range;
 * wsic_debug_get writes the current value to *value (host); wsic_debug_reset restores every
 * default.
 */
enum wsic_debug_knob {
  WSIC_DBG_FP64_PRODUCT = 0,
  WSIC_DBG_SUPER_BLOCKS = 1,
  WSIC_DBG_GUARD_SCALE = 2,
  WSIC_DBG_CHOL_FUSED = 3,
  WSIC_DBG_LOGITS_GENERIC = 4,
  WSIC_DBG_TRACE = 5,
  WSIC_DBG_PROBE = 6
};
int wsic_debug_set(int knob, double value);
int wsic_debug_get(int knob, double* value);
void wsic_debug_reset(void);

/*
 * Kernel timing. While enabled, every kernel launch is bracketed by HIP events on its own
 * stream; wsic_profile_read synchronizes and returns, for the kernel family `name`, the
 * launch count, the summed event time in ms and the summed algorithmic work (flops for the
 * MFMA kernels, bytes for the streaming kernels). wsic_profile_names writes a
 * comma-separated list of the families seen into buf. wsic_profile_select restricts the timing
 * to the families in a comma-separated list (NULL or "" = every family), so that the events
 * disturb nothing else. Not thread-safe.
 */
int wsic_profile_enable(int on);
int wsic_profile_select(const char* families);
int wsic_profile_reset(void);
int wsic_profile_read(const char* name, int64_t* launches, double* total_ms, double* total_work);
int wsic_profile_names(char* buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif
#endif /* WSIC_H */
