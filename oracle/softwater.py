"""fp64 oracle for SoftWater (class-aware rate allocation of a softmax output layer).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module. It shares no code with the HIP path.

Source: the web page "SoftWater: Class-Aware Rate Allocation for Softmax Quantization"
(Portuguese technical summary), cited below as [SoftWater, <section>]:
  * §2 "Derivação do Objetivo": the distortion of a quantized softmax layer is the expected
    KL divergence between the original and the quantized output distributions; to second
    order in the logit perturbation it is 1/2 vec(Delta)^T E[H(p) (x) x x^T] vec(Delta) with
    H(p) = diag(p) - p p^T the softmax Hessian.
  * §2 "Aproximação Tratável": subtractive dither drops the off-diagonal Hessian terms
    (errors uncorrelated across rows); separability factors the expectation as
    E[lambda] (x) E[x x^T]. The grid step of class k and input column i is then
    proportional to 1 / (lambda_bar_k^(1/2) |l_ii|), lambda_bar_k = E[p_k (1 - p_k)].
  * §2 "Prior de Suavização": the calibration distribution is mixed with a uniform one so
    that lambda_bar_k stays away from zero for classes the calibration data never predicts,
    bounding the largest grid step.
  * §2 "Implementação": the codes come from SIC as in WaterSIC, with the class-specific
    rescaling; one forward pass over the calibration data gives Sigma_X and lambda_bar.

Readings taken where the page is silent (each also listed in the design notes):
  * The smoothing prior mixes every calibration softmax output with the uniform
    distribution over the K classes: p~ = (1 - eps) p + eps / K, and lambda_bar_k is the
    calibration mean of p~_k (1 - p~_k). The weight eps is a parameter (eps = 0: none).
  * Rows of W are classes (W is K x n, logits W x). The grid of weight (k, j) is
    c / (sqrt(lambda_bar_k) |l_jj|) with one global scale c, SIC visits the columns in the
    WaterSIC order, and the rate is the pooled empirical entropy of all codes, so c is found
    by the same controller as WaterSIC (``watersic.waterfill``).
  * The distortion reported is the separable second-order KL estimate
    1/2 sum_k lambda_bar_k (e_k Sigma e_k^T) with e_k = w_k - w_hat_k, Sigma = X^T X / N.

Parity status: every function is pinned by the CPU tests (closed forms for uniform outputs and
for two classes, the bounds the smoothing prior implies, per-row reduction to the WaterSIC
oracle, agreement of the second-order form with the exact KL divergence for small
perturbations, the residual identity).
"""
from __future__ import annotations

from typing import Dict, Iterable

import numpy as np

from . import watersic

__all__ = [
    "softmax_probs",
    "softmax_curvature",
    "grid_steps",
    "sic_quantize",
    "initial_scale",
    "waterfill",
    "kl_distortion",
    "kl_distortion_from_residuals",
    "kl_second_order",
    "kl_exact",
]


def softmax_probs(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Row n of the result is softmax(W x_n) over the K classes, in fp64 (the max logit is
    subtracted before exponentiating)."""
    logits = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


def softmax_curvature(x_chunks: Iterable[np.ndarray], W: np.ndarray, smoothing: float = 0.0,
                      rows_per_step: int = 256) -> np.ndarray:
    """lambda_bar_k = mean over calibration rows x_n of p~_k (1 - p~_k) [SoftWater, §2
    "Aproximação Tratável"], with p~ = (1 - eps) softmax(W x_n) + eps / K the output mixed
    with the uniform distribution [§2 "Prior de Suavização"]."""
    W64 = np.asarray(W, dtype=np.float64)
    K = W64.shape[0]
    eps = float(smoothing)
    acc = np.zeros(K)
    n = 0
    for X in x_chunks:
        X = np.asarray(X)
        for r0 in range(0, X.shape[0], rows_per_step):
            p = softmax_probs(X[r0:r0 + rows_per_step], W64)
            pt = (1.0 - eps) * p + eps / K
            acc += (pt * (1.0 - pt)).sum(axis=0)
        n += X.shape[0]
    return acc / n


def grid_steps(L: np.ndarray, lam: np.ndarray, c: float) -> np.ndarray:
    """alpha_kj = c / (sqrt(lambda_bar_k) |l_jj|) [SoftWater, §2 "Aproximação Tratável"]:
    one global constant c, finer grids for classes of larger curvature."""
    return c / (np.sqrt(np.asarray(lam, dtype=np.float64))[:, None] * np.abs(np.diag(L))[None, :])


def sic_quantize(W: np.ndarray, L: np.ndarray, lam: np.ndarray, c: float) -> Dict[str, np.ndarray]:
    """SIC with the class-specific grids [SoftWater, §2 "Implementação"]: the WaterSIC
    recursion (columns j = n-1 ... 0, interference of the quantized columns cancelled with
    weights L_kj / l_jj) where row k rounds on its own step alpha_kj.

    Returns q (int64), t (targets), r (residuals t - alpha q), e (raw errors), alpha (K x n)."""
    W64 = np.asarray(W, dtype=np.float64)
    K, n = W64.shape
    alpha = grid_steps(L, lam, c)
    g = L / np.diag(L)[None, :]
    eT = np.zeros((n, K))
    q = np.zeros((K, n), dtype=np.int64)
    t = np.zeros((K, n))
    r = np.zeros((K, n))
    for j in range(n - 1, -1, -1):
        tj = W64[:, j] + g[j + 1:, j] @ eT[j + 1:, :]
        qj = np.rint(tj / alpha[:, j])
        eT[j, :] = W64[:, j] - alpha[:, j] * qj
        t[:, j] = tj
        r[:, j] = tj - alpha[:, j] * qj
        q[:, j] = qj.astype(np.int64)
    return {"q": q, "t": t, "r": r, "e": eT.T.copy(), "alpha": alpha}


def initial_scale(W: np.ndarray, L: np.ndarray, lam: np.ndarray, rate: float) -> float:
    """High-rate start of the search: the WaterSIC estimate for the rows w_k sqrt(lambda_k),
    whose grids c / |l_jj| are those of row k."""
    Ws = np.asarray(W, dtype=np.float64) * np.sqrt(np.asarray(lam, dtype=np.float64))[:, None]
    return watersic.initial_scale(Ws, L, rate)


def waterfill(W: np.ndarray, L: np.ndarray, lam: np.ndarray, rate: float, **kw) -> Dict[str, object]:
    """The smallest c with pooled code entropy <= rate, found by the WaterSIC controller
    (bracketing, then geometric bisection) over the class-aware SIC."""
    return watersic.waterfill(W, L, rate, quantize=lambda c: sic_quantize(W, L, lam, c),
                              c_start=initial_scale(W, L, lam, rate), **kw)


def kl_distortion(W: np.ndarray, q: np.ndarray, alpha: np.ndarray, sigma: np.ndarray,
                  lam: np.ndarray) -> float:
    """1/2 sum_k lambda_bar_k e_k Sigma e_k^T, e = W - q * alpha: the second-order KL
    divergence after the dither and separability approximations [SoftWater, §2]."""
    E = np.asarray(W, dtype=np.float64) - np.asarray(q, dtype=np.float64) * alpha
    per_row = np.sum(E * (E @ np.asarray(sigma, dtype=np.float64)), axis=1)
    return 0.5 * float(np.dot(np.asarray(lam, dtype=np.float64), per_row))


def kl_distortion_from_residuals(r: np.ndarray, L: np.ndarray, lam: np.ndarray) -> float:
    """The same estimate from the SIC residuals: 1/2 sum_k lambda_k sum_j l_jj^2 r_kj^2 (the
    whitened error of column j of row k is l_jj r_kj, as in WaterSIC)."""
    r = np.asarray(r, dtype=np.float64)
    w = (np.diag(L) ** 2)[None, :] * r * r
    return 0.5 * float(np.dot(np.asarray(lam, dtype=np.float64), w.sum(axis=1)))


def kl_second_order(X: np.ndarray, W: np.ndarray, W_hat: np.ndarray) -> float:
    """Mean over rows x_n of 1/2 d^T (diag(p) - p p^T) d, d = (W - W_hat) x_n, p = softmax(W x_n):
    the second-order form before any approximation [SoftWater, §2 "Derivação do Objetivo"]."""
    p = softmax_probs(X, W)
    D = np.asarray(X, dtype=np.float64) @ (np.asarray(W, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)).T
    quad = np.sum(p * D * D, axis=1) - np.sum(p * D, axis=1) ** 2
    return 0.5 * float(quad.mean())


def kl_exact(X: np.ndarray, W: np.ndarray, W_hat: np.ndarray) -> float:
    """Mean over rows of KL(softmax(W x) || softmax(W_hat x)), the distortion itself."""
    p = softmax_probs(X, W)
    qh = softmax_probs(X, W_hat)
    return float(np.mean(np.sum(p * (np.log(p) - np.log(qh)), axis=1)))
