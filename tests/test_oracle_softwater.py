"""Pins of the SoftWater oracle (CPU only): closed forms, bounds, reductions to the WaterSIC
oracle and to the exact KL divergence. Each test names the passage of the SoftWater page
("SoftWater: Class-Aware Rate Allocation for Softmax Quantization", §2) it checks."""
import math

import numpy as np
import pytest

from oracle import softwater as sw
from oracle import watersic as ws


def _problem(seed=0, rows=400, n=10, K=7, wscale=0.4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((rows, n)) * np.exp(0.3 * rng.standard_normal(n))[None, :]
    W = rng.standard_normal((K, n)) * wscale
    L, info = ws.cholesky_lower(ws.covariance([X]))
    assert info == 0
    return X, W, L


@pytest.mark.parametrize("eps", [0.0, 0.05, 0.5])
def test_curvature_uniform_outputs(eps):
    """Identical class rows give the uniform softmax for every input, so
    lambda_k = (1/K)(1 - 1/K) whatever the smoothing (§2 "Aproximação Tratável")."""
    X, W, _ = _problem()
    K = W.shape[0]
    Wsame = np.repeat(W[:1], K, axis=0)
    lam = sw.softmax_curvature([X], Wsame, eps)
    np.testing.assert_allclose(lam, (1 / K) * (1 - 1 / K), rtol=1e-14)


def test_curvature_full_smoothing_is_uniform():
    """eps = 1 replaces every output by the uniform distribution (§2 "Prior de Suavização")."""
    X, W, _ = _problem()
    K = W.shape[0]
    np.testing.assert_allclose(sw.softmax_curvature([X], W, 1.0), (1 / K) * (1 - 1 / K), rtol=1e-13)


def test_curvature_two_classes_is_logistic():
    """K = 2: p_1 = sigmoid((w_1 - w_2) x), so both curvatures equal mean sigma (1 - sigma)."""
    X, W, _ = _problem(K=2)
    d = X @ (W[0] - W[1])
    s = np.array([1.0 / (1.0 + math.exp(-v)) for v in d])
    ref = float(np.mean(s * (1.0 - s)))
    lam = sw.softmax_curvature([X], W)
    np.testing.assert_allclose(lam, [ref, ref], rtol=1e-12)


def test_curvature_brute_force_loops():
    """Pure-Python loops over samples and classes (logit of class k = sum_i W[k, i] x_i) with
    the smoothing mix, against the vectorized oracle, on ragged chunks."""
    X, W, _ = _problem(rows=37, n=5, K=4)
    eps = 0.2
    K = W.shape[0]
    acc = [0.0] * K
    for x in X:
        logit = [sum(W[k, i] * x[i] for i in range(W.shape[1])) for k in range(K)]
        m = max(logit)
        e = [math.exp(v - m) for v in logit]
        z = sum(e)
        for k in range(K):
            pt = (1 - eps) * e[k] / z + eps / K
            acc[k] += pt * (1 - pt)
    ref = np.array(acc) / X.shape[0]
    lam = sw.softmax_curvature([X[:10], X[10:11], X[11:]], W, eps, rows_per_step=4)
    np.testing.assert_allclose(lam, ref, rtol=1e-12)


@pytest.mark.parametrize("eps", [0.0, 0.01, 0.3])
def test_curvature_bounds(eps):
    """0 < lambda_k <= 1/4; sum_k lambda_k = 1 - E sum_k p~_k^2 <= 1 - 1/K; with smoothing,
    p~_k lies in [eps/K, 1 - eps + eps/K], which bounds lambda_k from below and so the largest
    grid step (§2 "Prior de Suavização")."""
    X, W, _ = _problem(wscale=3.0, K=9)
    K = W.shape[0]
    lam = sw.softmax_curvature([X], W, eps)
    assert np.all(lam > 0) and np.all(lam <= 0.25 + 1e-15)
    assert lam.sum() <= 1 - 1 / K + 1e-12
    if eps > 0:
        a, b = eps / K, 1 - eps + eps / K
        assert np.all(lam >= min(a * (1 - a), b * (1 - b)) - 1e-15)


def test_sic_rows_reduce_to_watersic():
    """Each row k is the WaterSIC SIC of that row alone at scale c / sqrt(lambda_k): the
    class-specific grid only rescales row k's steps (§2 "Implementação")."""
    X, W, L = _problem(K=6)
    lam = np.array([0.01, 0.2, 0.05, 0.11, 0.003, 0.24])
    c = 0.05
    res = sw.sic_quantize(W, L, lam, c)
    for k in range(W.shape[0]):
        one = ws.sic_quantize(W[k:k + 1], L, c / math.sqrt(lam[k]))
        np.testing.assert_array_equal(res["q"][k], one["q"][0])
        np.testing.assert_allclose(res["r"][k], one["r"][0], rtol=1e-12, atol=1e-15)


def test_sic_unit_curvature_is_watersic():
    X, W, L = _problem()
    c = 0.03
    a = sw.sic_quantize(W, L, np.ones(W.shape[0]), c)
    b = ws.sic_quantize(W, L, c)
    np.testing.assert_array_equal(a["q"], b["q"])
    np.testing.assert_array_equal(a["r"], b["r"])


def test_second_order_form_matches_exact_kl():
    """For a small logit perturbation the second-order form with the softmax Hessian
    diag(p) - p p^T equals the KL divergence to first order in its size (§2 "Derivação do
    Objetivo"): the ratio tends to 1 and the divergence scales quadratically."""
    X, W, _ = _problem()
    rng = np.random.default_rng(3)
    P = rng.standard_normal(W.shape)
    r = []
    for h in (1e-2, 1e-3):
        Wh = W + h * P
        r.append(sw.kl_second_order(X, W, Wh) / sw.kl_exact(X, W, Wh))
    assert abs(r[1] - 1) < 2e-3 and abs(r[1] - 1) < abs(r[0] - 1)
    k1 = sw.kl_exact(X, W, W + 1e-3 * P)
    k2 = sw.kl_exact(X, W, W + 2e-3 * P)
    assert abs(k2 / k1 - 4) < 2e-2


def test_separable_form_is_exact_for_constant_outputs():
    """When p does not depend on the input (identical class rows), the dithered form
    1/2 E[sum_k p_k (1 - p_k) d_k^2] factors exactly into 1/2 sum_k lambda_k e_k Sigma e_k^T
    (§2 "Aproximação Tratável")."""
    X, W, _ = _problem()
    K = W.shape[0]
    Wsame = np.repeat(W[:1], K, axis=0)
    lam = sw.softmax_curvature([X], Wsame)
    E = np.random.default_rng(4).standard_normal(W.shape) * 1e-2
    sigma = ws.covariance([X])
    sep = sw.kl_distortion(E, np.zeros(W.shape), np.zeros(W.shape), sigma, lam)
    p = sw.softmax_probs(X, Wsame)
    d = X @ E.T
    dithered = 0.5 * float(np.mean(np.sum(p * (1 - p) * d * d, axis=1)))
    np.testing.assert_allclose(sep, dithered, rtol=1e-12)


def test_kl_distortion_residual_identity():
    """1/2 sum_k lambda_k e_k Sigma e_k^T equals 1/2 sum_k lambda_k sum_j l_jj^2 r_kj^2 for the
    SIC output (Sigma = L L^T)."""
    X, W, L = _problem(K=5)
    lam = sw.softmax_curvature([X], W, 0.05)
    res = sw.sic_quantize(W, L, lam, 0.02)
    sigma = L @ L.T
    d1 = sw.kl_distortion(W, res["q"], res["alpha"], sigma, lam)
    d2 = sw.kl_distortion_from_residuals(res["r"], L, lam)
    np.testing.assert_allclose(d1, d2, rtol=1e-10)
    # every residual within half its own step
    assert np.all(np.abs(res["r"]) <= res["alpha"] / 2 * (1 + 1e-12))


def test_waterfill_unit_curvature_is_watersic():
    X, W, L = _problem(rows=500, n=12, K=20)
    a = sw.waterfill(W, L, np.ones(W.shape[0]), 2.0)
    b = ws.waterfill(W, L, 2.0)
    assert a["c"] == b["c"] and a["rate"] == b["rate"]


def test_waterfill_budget():
    X, W, L = _problem(rows=500, n=12, K=20)
    lam = sw.softmax_curvature([X], W, 0.05)
    wf = sw.waterfill(W, L, lam, 1.5)
    assert wf["rate"] <= 1.5
    assert ws.entropy_bits(wf["sic"]["q"]) == wf["rate"]
    # the next grid scale below the bracket exceeds the budget
    lo = sw.sic_quantize(W, L, lam, wf["c_lo"])
    assert ws.entropy_bits(lo["q"]) > 1.5
