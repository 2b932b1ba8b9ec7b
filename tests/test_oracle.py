"""Pins of the fp64 oracle against what the WaterSIC page and the mathematics fix.

Each test checks the oracle against something other than itself: a hand-worked example
(tests/golden), a closed form, a brute-force search, a library routine, an exact invariance,
or the page's 0.255-bit rate gap.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from golden_io import load
from rate_allocated_weight_amd import workloads


def _rng(seed):
    return np.random.default_rng(seed)


def _ar1_sigma(n, rho):
    idx = np.arange(n)
    return rho ** np.abs(idx[:, None] - idx[None, :])


def _random_spd(rng, n, cond=100.0):
    q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    ev = np.exp(rng.uniform(0, math.log(cond), n))
    return (q * ev) @ q.T


# ---------------------------------------------------------------- hand-worked examples
@pytest.mark.parametrize("name", ["hand_sic_2x2.txt", "hand_sic_3x3.txt"])
def test_hand_worked_sic(name):
    g = load(name)
    W = np.atleast_2d(g["W"])
    L, info = oracle.cholesky_lower(g["sigma"])
    assert info == 0
    np.testing.assert_array_equal(L, g["L"])  # exact: all entries are small integers
    res = oracle.sic_quantize(W, L, g["c"])
    np.testing.assert_array_equal(res["alpha"], g["alpha"])
    np.testing.assert_array_equal(res["q"], np.atleast_2d(g["q"]).astype(np.int64))
    np.testing.assert_array_equal(res["t"], np.atleast_2d(g["t"]))
    np.testing.assert_array_equal(res["r"], np.atleast_2d(g["r"]))
    np.testing.assert_array_equal(res["e"], np.atleast_2d(g["e"]))
    assert oracle.distortion_direct(W, res["q"], res["alpha"], g["sigma"]) == g["D"]
    assert oracle.distortion_from_residuals(res["r"], L) == g["D"]
    np.testing.assert_array_equal(oracle.babai_codes(W, L, g["c"]), res["q"])


def test_hand_covariance_and_factor():
    g = load("hand_covariance.txt")
    sigma = oracle.covariance([g["X"]])
    np.testing.assert_array_equal(sigma, g["sigma"])
    L, info = oracle.cholesky_lower(sigma)
    assert info == 0
    np.testing.assert_allclose(L, g["L"], rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- covariance
def test_covariance_chunking_and_orthogonal_rows():
    rng = _rng(1)
    X = rng.standard_normal((97, 13))
    whole = oracle.covariance([X])
    parts = oracle.covariance([X[:40], X[40:41], X[41:]])
    np.testing.assert_allclose(parts, whole, rtol=1e-13, atol=1e-15)
    # rows of sqrt(N) * an orthogonal matrix give the identity exactly up to rounding
    q, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    np.testing.assert_allclose(oracle.covariance([4.0 * q]), np.eye(16), atol=1e-14)


def test_covariance_entries_match_the_whole_matrix():
    rng = np.random.default_rng(11)
    chunks = [rng.standard_normal((r, 24)).astype(np.float32) for r in (7, 1, 30)]
    whole = oracle.covariance(chunks)
    I = rng.integers(0, 24, 50)
    J = rng.integers(0, 24, 50)
    np.testing.assert_allclose(oracle.covariance_entries(chunks, I, J), whole[I, J], rtol=1e-13, atol=1e-15)
    # a single calibration row: x_i x_j exactly
    x = np.array([[0.5, -2.0, 3.0]], dtype=np.float32)
    assert oracle.covariance_entries([x], np.array([0, 1, 2]), np.array([2, 1, 0])).tolist() == [1.5, 4.0, 1.5]


def test_covariance_matches_population_ar1():
    # AR(1) rows from the workload generator: Sigma_ij -> rho^|i-j| as N grows
    lay = workloads.make_layer("ar1", 4, 24, 200000, dtype="f32", rho=0.9, seed=3)
    sigma = oracle.covariance(lay.x_chunks)
    assert np.max(np.abs(sigma - _ar1_sigma(24, 0.9))) < 0.03


# ---------------------------------------------------------------- Cholesky
@pytest.mark.parametrize("n", [1, 2, 7, 64, 200])
def test_cholesky_textbook_vs_lapack(n):
    rng = _rng(n)
    A = _random_spd(rng, n, cond=1e4)
    L1, i1 = oracle.cholesky_lower_textbook(A)
    assert i1 == 0
    L2 = np.linalg.cholesky(A)
    np.testing.assert_allclose(L1, L2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(L1 @ L1.T, A, rtol=1e-12, atol=1e-12)
    assert np.all(np.diag(L1) > 0) and np.allclose(np.triu(L1, 1), 0)


def test_cholesky_large_path_and_ar1_closed_form():
    # AR(1): x_0 = z_0, x_i = rho x_{i-1} + s z_i gives L_ij = rho^(i-j) s_j, s_0 = 1
    n, rho = 300, 0.9
    s = np.full(n, math.sqrt(1 - rho * rho))
    s[0] = 1.0
    i, j = np.indices((n, n))
    L_exact = np.where(i >= j, rho ** (i - j).clip(0) * s[None, :], 0.0)
    L, info = oracle.cholesky_lower(_ar1_sigma(n, rho))  # n > 256: LAPACK route
    assert info == 0
    np.testing.assert_allclose(L, L_exact, atol=1e-12)


@pytest.mark.parametrize("n,bad", [(5, 3), (300, 117)])
def test_cholesky_reports_failing_pivot(n, bad):
    A = _ar1_sigma(n, 0.5)
    A[bad - 1, :] = 0.0
    A[:, bad - 1] = 0.0
    L, info = oracle.cholesky_lower(A)
    assert L is None and info == bad


# ---------------------------------------------------------------- SIC special cases
def test_identity_covariance_is_round_to_nearest():
    rng = _rng(2)
    W = rng.standard_normal((37, 11))
    c = 0.3
    res = oracle.sic_quantize(W, np.eye(11), c)
    np.testing.assert_array_equal(res["q"], np.rint(W / c).astype(np.int64))


def test_diagonal_covariance_is_per_column_rtn():
    rng = _rng(3)
    W = rng.standard_normal((29, 9))
    dvar = np.exp(rng.standard_normal(9))
    L = np.diag(np.sqrt(dvar))
    c = 0.7
    res = oracle.sic_quantize(W, L, c)
    step = c / np.sqrt(dvar)
    np.testing.assert_array_equal(res["q"], np.rint(W / step[None, :]).astype(np.int64))


def test_residual_bound_and_babai_equivalence():
    rng = _rng(4)
    for n_out, n in [(50, 1), (40, 6), (33, 40)]:
        A = _random_spd(rng, n, cond=1e3)
        L, _ = oracle.cholesky_lower(A)
        W = rng.standard_normal((n_out, n)) * 0.1
        for c in (0.02, 0.3):
            res = oracle.sic_quantize(W, L, c)
            assert np.all(np.abs(res["r"]) <= res["alpha"][None, :] * (0.5 + 1e-12))
            np.testing.assert_array_equal(oracle.babai_codes(W, L, c), res["q"])


def test_distortion_identity_random():
    rng = _rng(5)
    A = _random_spd(rng, 30, cond=1e5)
    L, _ = oracle.cholesky_lower(A)
    W = rng.standard_normal((20, 30))
    res = oracle.sic_quantize(W, L, 0.4)
    d1 = oracle.distortion_direct(W, res["q"], res["alpha"], A)
    d2 = oracle.distortion_from_residuals(res["r"], L)
    assert abs(d1 - d2) <= 1e-12 * d1


def test_high_rate_distortion():
    # At high rate each whitened residual is ~uniform on [-c/2, c/2]: D ~ N_p c^2 / 12
    rng = _rng(6)
    A = _ar1_sigma(16, 0.9)
    L, _ = oracle.cholesky_lower(A)
    W = rng.standard_normal((4000, 16))
    c = 0.01  # ~8 bits per weight here
    res = oracle.sic_quantize(W, L, c)
    D = oracle.distortion_direct(W, res["q"], res["alpha"], A)
    ratio = D / (W.size * c * c / 12.0)
    assert 0.98 < ratio < 1.02
    per_col = (np.diag(L) ** 2) * (res["r"] ** 2).sum(axis=0)
    np.testing.assert_allclose(per_col / (4000 * c * c / 12.0), 1.0, atol=0.08)


@pytest.mark.parametrize("n", [1, 2, 3])
def test_brute_force_babai_cell_and_cvp(n):
    """SIC codes are the unique q whose whitened error lies in the box |(e L)_j| <= c/2;
    the exact closest lattice point is never worse, and equals SIC for n = 1 / diagonal."""
    rng = _rng(10 + n)
    grid = np.arange(-14, 15)
    for trial in range(4):
        diag_case = trial == 3
        if diag_case:
            A = np.diag(np.exp(rng.standard_normal(n)))
        else:
            A = _random_spd(rng, n, cond=30.0)
        L, _ = oracle.cholesky_lower(A)
        W = rng.standard_normal((25, n)) * 0.5
        c = 0.6
        res = oracle.sic_quantize(W, L, c)
        assert np.abs(res["q"]).max() < 14  # the search box holds every SIC code
        alpha = res["alpha"]
        cands = np.array(list(itertools.product(grid, repeat=n)), dtype=np.float64)
        for r in range(W.shape[0]):
            E = W[r][None, :] - cands * alpha[None, :]
            white = E @ L  # row-wise (e L)
            inbox = np.all(np.abs(white) <= c / 2 + 1e-12, axis=1)
            assert inbox.sum() == 1
            np.testing.assert_array_equal(cands[inbox][0].astype(np.int64), res["q"][r])
            dist = np.sum(white * white, axis=1)
            d_sic = dist[inbox][0]
            assert dist.min() <= d_sic + 1e-15
            if n == 1 or diag_case:
                assert dist.min() == pytest.approx(d_sic, rel=1e-12, abs=1e-15)


def test_exact_power_of_two_invariances_and_row_permutation():
    rng = _rng(7)
    A = _random_spd(rng, 24, cond=1e3)
    L, _ = oracle.cholesky_lower(A)
    W = rng.standard_normal((31, 24))
    c = 0.25
    q = oracle.sic_quantize(W, L, c)["q"]
    np.testing.assert_array_equal(oracle.sic_quantize(4.0 * W, L, 4.0 * c)["q"], q)
    L4, _ = oracle.cholesky_lower(16.0 * A)  # L -> 4 L, alpha -> alpha/4 at the same c
    np.testing.assert_array_equal(oracle.sic_quantize(W, L4, 4.0 * c)["q"], q)
    perm = rng.permutation(31)
    np.testing.assert_array_equal(oracle.sic_quantize(W[perm], L, c)["q"], q[perm])


def test_interference_changes_codes():
    # Guards against a variant that drops the cancellation term or runs forward
    rng = _rng(8)
    A = _ar1_sigma(32, 0.95)
    L, _ = oracle.cholesky_lower(A)
    W = rng.standard_normal((64, 32))
    c = 0.5
    q = oracle.sic_quantize(W, L, c)["q"]
    rtn = np.rint(W / oracle.grid_steps(L, c)[None, :]).astype(np.int64)
    assert np.mean(q != rtn) > 0.05
    # reverse order: quantizing the column-reversed problem with the factor of the reversed
    # covariance (a forward SIC in disguise) gives different codes
    Ar = A[::-1, ::-1]
    Lr, _ = oracle.cholesky_lower(Ar)
    qf = oracle.sic_quantize(W[:, ::-1], Lr, c)["q"][:, ::-1]
    assert np.mean(qf != q) > 0.01


# ---------------------------------------------------------------- entropy
def test_entropy_closed_forms():
    assert oracle.entropy_bits(np.zeros(100, dtype=np.int64)) == 0.0
    for k in range(1, 6):
        codes = np.repeat(np.arange(-(2 ** (k - 1)), 2 ** (k - 1)), 3)
        assert oracle.entropy_bits(codes) == pytest.approx(k, abs=1e-15)
    h = oracle.entropy_bits(np.array([0, 0, 0, 1]))
    assert h == pytest.approx(-(0.75 * math.log2(0.75) + 0.25 * math.log2(0.25)), abs=1e-15)
    assert oracle.entropy_bits(np.array([], dtype=np.int64)) == 0.0
    # unbounded integers count as symbols like any other
    assert oracle.entropy_bits(np.array([-(2 ** 40), 2 ** 40])) == pytest.approx(1.0)


def test_rate_gap_matches_page_constant():
    """[WaterSIC §3]: at high rate WaterSIC's rate exceeds the Gaussian rate-distortion
    function by 0.5*log2(2 pi e/12) = 0.255 bit, for any covariance."""
    g = load("page_constants.txt")
    assert oracle.RATE_GAP_BITS == pytest.approx(g["rate_gap_bits_printed"], abs=5e-4)
    rng = _rng(9)
    n = 8
    dsc = np.exp(0.5 * rng.standard_normal(n))
    A = _ar1_sigma(n, 0.9) * dsc[:, None] * dsc[None, :]
    L, _ = oracle.cholesky_lower(A)
    W = rng.standard_normal((40000, n))  # iid unit-variance Gaussian weights
    c = 0.08
    res = oracle.sic_quantize(W, L, c)
    h_cols = np.mean([oracle.entropy_bits(res["q"][:, j]) for j in range(n)])
    D = oracle.distortion_from_residuals(res["r"], L) / W.shape[0]  # per row
    # reverse waterfilling on the eigenvalues of the whitened source covariance
    mu = np.linalg.eigvalsh(A)
    theta = D / n
    assert theta < mu.min()  # high-rate regime: every component is active
    r_it = 0.5 * np.sum(np.log2(mu / theta)) / n
    assert h_cols - r_it == pytest.approx(oracle.RATE_GAP_BITS, abs=0.03)
    # the same budget spent on one uniform step for every column is farther from the limit
    step = np.full(n, np.exp(np.mean(np.log(res["alpha"]))))
    L_id = np.eye(n)
    q_u = np.rint(W / step[None, :])
    e_u = W - q_u * step[None, :]
    D_u = np.sum(e_u * (e_u @ A)) / W.shape[0]
    h_u = np.mean([oracle.entropy_bits(q_u[:, j]) for j in range(n)])
    r_it_u = 0.5 * np.sum(np.log2(mu / (D_u / n))) / n if D_u / n < mu.min() else None
    assert r_it_u is not None and (h_u - r_it_u) > oracle.RATE_GAP_BITS + 0.05
    del L_id


# ---------------------------------------------------------------- controller
def test_controller_brackets_crossing_against_scan():
    rng = _rng(11)
    A = _ar1_sigma(3, 0.9)
    L, _ = oracle.cholesky_lower(A)
    W = rng.standard_normal((64, 3)) * 0.02
    R = 2.0
    wf = oracle.waterfill(W, L, R)
    c = wf["c"]
    assert wf["rate"] <= R
    assert oracle.entropy_bits(oracle.sic_quantize(W, L, wf["c_lo"])["q"]) > R
    assert math.log2(c / wf["c_lo"]) <= 2.0 ** -20
    # dense scan of H(c): the crossing nearest below c must be within the bracket
    cs = c * 2.0 ** np.linspace(-0.5, 0.5, 4001)
    hs = np.array([oracle.entropy_bits(oracle.sic_quantize(W, L, x)["q"]) for x in cs])
    ok = hs <= R
    # every scanned point with c' <= c_lo has H > R unless H is non-monotone there
    first_ok = cs[np.argmax(ok)]
    assert first_ok >= wf["c_lo"] * (1 - 1e-9) or np.any(~ok[cs > first_ok])
    # the smallest grid point at or above c satisfies the budget
    assert hs[np.searchsorted(cs, c)] <= R


def test_controller_hits_rate_on_small_layer():
    lay = workloads.named_workload("ar1_256")
    sigma = oracle.covariance(lay.x_chunks)
    L, info = oracle.cholesky_lower(sigma)
    assert info == 0
    W = lay.w[:64]
    wf = oracle.waterfill(W, L, 2.0)
    assert 2.0 - 1e-3 < wf["rate"] <= 2.0
    hs = [h for _, h in wf["trace"]]
    assert len(hs) < 60


def test_quantize_layer_end_to_end_small():
    lay = workloads.make_layer("spiked", 40, 48, 300, dtype="bf16", rank=8, seed=2)
    out = oracle.quantize_layer(lay.w, lay.x_chunks, 2.0)
    assert out["rate"] <= 2.0
    assert out["D"] == pytest.approx(out["D_resid"], rel=1e-10)


# ------------------------------------------------------------------ per-column rate and the limit
def test_entropy_columns_closed_forms():
    """Each column uniform over 2^k symbols has k bits; a constant column has 0; the pooled
    entropy is at least the mean column entropy (concavity of entropy under mixing)."""
    rng = np.random.default_rng(0)
    k = [1, 3, 0, 5]
    cols = []
    for kk in k:
        v = np.repeat(np.arange(2 ** kk), 64 // 2 ** kk * 4)[:256] + 7 * kk
        cols.append(rng.permutation(v))
    q = np.stack(cols, axis=1)
    assert oracle.entropy_bits_columns(q) == pytest.approx(np.mean(k), abs=1e-12)
    r = rng.integers(-6, 7, size=(500, 9)) * rng.integers(1, 4, size=9)[None, :]
    assert oracle.entropy_bits(r) >= oracle.entropy_bits_columns(r) - 1e-12


def test_gaussian_rate_identity_and_zero():
    """Sigma = I: R(D) = 1/2 log2(var / D) for D < var, 0 beyond."""
    mu = np.ones(7)
    for D in (0.01, 0.3, 0.9):
        assert oracle.gaussian_rate(mu, 1.3, D) == pytest.approx(0.5 * np.log2(1.3 / D), rel=1e-12)
    assert oracle.gaussian_rate(mu, 1.3, 1.3) == 0.0


def test_gaussian_rate_water_level_by_hand():
    """mu = (1, 0.01), var 1, D = 0.1 per weight: the water level theta solves
    (min(theta, 1) + min(theta, 0.01)) / 2 = 0.1, theta = 0.19; only the first component is
    coded: R = (1/2)(1/2) log2(1 / 0.19)."""
    r = oracle.gaussian_rate(np.array([1.0, 0.01]), 1.0, 0.1)
    assert r == pytest.approx(0.25 * np.log2(1.0 / 0.19), rel=1e-10)


def test_gaussian_rate_high_rate_is_log_det():
    """Below the smallest eigenvalue the water level is D itself and the rate is
    1/2 log2(var/D) + (1/n) sum_j log2 l_jj (det Sigma from the Cholesky diagonal)."""
    rng = np.random.default_rng(1)
    A = rng.standard_normal((10, 10))
    sigma = A @ A.T + 0.5 * np.eye(10)
    L, info = oracle.cholesky_lower(sigma)
    mu = np.linalg.eigvalsh(sigma)
    D = 0.1 * 0.7 * mu.min()
    assert oracle.gaussian_rate(mu, 0.7, D) == pytest.approx(oracle.gaussian_rate_high(np.diag(L), 0.7, D),
                                                             rel=1e-10)


def test_watersic_gap_at_high_rate():
    """[WaterSIC, §3 Limiti teorici]: with per-column entropy coding the rate of WaterSIC sits
    1/2 log2(2 pi e / 12) = 0.2546 bit above the Gaussian limit at high rate (sanity, +-0.03)."""
    rng = np.random.default_rng(5)
    n = 12
    sigma = 0.9 ** np.abs(np.subtract.outer(np.arange(n), np.arange(n)))
    L, info = oracle.cholesky_lower(sigma)
    var_w = 0.02 ** 2
    W = rng.standard_normal((20000, n)) * np.sqrt(var_w)
    c = 2.0 ** -5 * 0.02
    res = oracle.sic_quantize(W, L, c)
    R = oracle.entropy_bits_columns(res["q"])
    D = oracle.distortion_from_residuals(res["r"], L) / W.size
    gap = R - oracle.gaussian_rate(np.linalg.eigvalsh(sigma), var_w, D)
    assert 4.0 < R < 8.0
    assert gap == pytest.approx(0.5 * np.log2(2 * np.pi * np.e / 12), abs=0.03)


# ------------------------------------------------------------------ LMMSE rescale
def _spd(n, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((n, n))
    return A @ A.T / n + 0.1 * np.eye(n)


def test_lmmse_scale_closed_forms():
    """gamma = 1 and no distortion when W_hat = W; W_hat = 2 W gives gamma = 1/2 and zero
    distortion after rescaling; a zero row keeps gamma = 1 and its distortion."""
    rng = np.random.default_rng(0)
    S = _spd(6, 1)
    W = rng.standard_normal((4, 6))
    r = oracle.lmmse_scale(W, W, S)
    np.testing.assert_allclose(r["gamma"], 1.0, rtol=1e-12)
    assert abs(r["D_after"]) < 1e-12
    r = oracle.lmmse_scale(W, 2 * W, S)
    np.testing.assert_allclose(r["gamma"], 0.5, rtol=1e-12)
    np.testing.assert_allclose(r["d_after"], 0.0, atol=1e-12)
    Wh = W.copy()
    Wh[2] = 0.0
    r = oracle.lmmse_scale(W, Wh, S)
    assert r["gamma"][2] == 1.0 and r["d_after"][2] == pytest.approx(W[2] @ S @ W[2])


def test_lmmse_scale_is_the_minimizer():
    """gamma_k minimizes the row's distortion over a scalar grid (brute force); never worse
    than gamma = 1; the before-distortion equals tr(E Sigma E^T) of the rows."""
    rng = np.random.default_rng(3)
    S = _spd(5, 2)
    W = rng.standard_normal((3, 5))
    Wh = np.rint(W * 2) / 2
    r = oracle.lmmse_scale(W, Wh, S)
    for k in range(3):
        g = np.linspace(r["gamma"][k] - 0.1, r["gamma"][k] + 0.1, 2001)
        d = [(W[k] - x * Wh[k]) @ S @ (W[k] - x * Wh[k]) for x in g]
        assert min(d) >= r["d_after"][k] - 1e-12
        assert r["d_after"][k] <= r["d_before"][k] + 1e-15
    assert r["D_before"] == pytest.approx(oracle.distortion_direct(W, Wh, np.ones(5), S), rel=1e-12)


def test_dead_features_removed_without_changing_the_distortion():
    """Columns of exactly zero variance make Sigma singular (the factorization fails); removing
    them leaves a factorable Sigma, and a dead column contributes nothing to tr(E Sigma E^T)
    whatever its weights, so the layer's distortion is that of the live problem."""
    rng = np.random.default_rng(2)
    X = rng.standard_normal((300, 9))
    X[:, [2, 6]] = 0.0
    sigma = oracle.covariance([X])
    L, info = oracle.cholesky_lower(sigma)
    assert info != 0
    live = oracle.live_features(sigma, 1e-12)
    np.testing.assert_array_equal(live, [0, 1, 3, 4, 5, 7, 8])
    S_l = sigma[np.ix_(live, live)]
    L_l, info = oracle.cholesky_lower(S_l)
    assert info == 0
    W = rng.standard_normal((5, 9))
    res = oracle.sic_quantize(W[:, live], L_l, 0.1)
    W_hat = np.zeros_like(W)
    W_hat[:, live] = res["q"] * res["alpha"][None, :]
    d_full = oracle.distortion_direct(W, W_hat, np.ones(9), sigma)
    d_live = oracle.distortion_from_residuals(res["r"], L_l)
    assert d_full == pytest.approx(d_live, rel=1e-10)
