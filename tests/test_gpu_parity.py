"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by element, at
sizes the oracle finishes in seconds: several 64/128-wide tiles and a ragged tail."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (DEV, RATE_TOL, REL_TOL, assert_codes_parity, say, w_tensor, x_tensors)
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu

LAYERS = {
    # name: (recipe, n_out, n_in, n_rows, kwargs)
    "ar1_256_f32": ("ar1", 256, 256, 1024, dict(dtype="f32", rho=0.9)),
    "spiked_300x333": ("spiked", 300, 333, 900, dict(dtype="bf16", rank=16)),
    "blockar1_77x520": ("blockar1", 77, 520, 1100, dict(dtype="bf16", block=96, chunk_rows=400)),
    "outliers_130x200": ("ar1", 130, 200, 600, dict(dtype="bf16", rho=0.95, scale_sigma=0.5,
                                                   outlier_cols=3)),
    # n_in a multiple of 16 but not of 128, n_out ragged: the pipelined Y product with partial tiles
    "spiked_200x272": ("spiked", 200, 272, 700, dict(dtype="bf16", rank=16)),
}


def _layer(name, seed=0):
    recipe, n_out, n_in, n_rows, kw = LAYERS[name]
    return workloads.make_layer(recipe, n_out, n_in, n_rows, seed=seed, name=name, **kw)


def _sigma_oracle(layer):
    return oracle.covariance(layer.x_chunks)


@pytest.fixture(scope="module")
def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.lib()
    return torch.device(DEV)


# ------------------------------------------------------------------ covariance
@pytest.mark.parametrize("name", list(LAYERS))
def test_covariance_parity(device, name):
    layer = _layer(name)
    say(f"[covariance] {name} rows={layer.n_rows} n_in={layer.n_in} chunks={len(layer.x_chunks)}")
    sig_gpu = lib.covariance_chunks(x_tensors(layer)).cpu().numpy()
    sig_or = _sigma_oracle(layer)
    scale = np.sqrt(np.outer(np.diag(sig_or), np.diag(sig_or)))
    err = np.max(np.abs(sig_gpu - sig_or) / scale)
    say(f"  max normalized |dSigma| = {err:.3e}")
    assert np.array_equal(sig_gpu, sig_gpu.T)
    tol = 1e-12 if layer.dtype == "f32" else 1e-6
    assert err <= tol


@pytest.mark.parametrize("n_in,rows", [(3072, 1000), (3000, 777)])
def test_covariance_split_tail_round(device, n_in, rows):
    """Widths whose tile count is not a multiple of the CU count: the tiles of the last, partial
    round are split along the calibration rows (here into pieces of a few 96-row steps, the last
    one ragged) and their partial sums added by a second launch. Also the streaming form
    (beta != 0) through the same path."""
    layer = workloads.make_layer("ar1", 8, n_in, rows, seed=11, name=f"split_{n_in}")
    say(f"[covariance-split] rows={rows} n_in={n_in}")
    X = x_tensors(layer)
    sig_gpu = lib.covariance_chunks(X).cpu().numpy()
    sig_or = _sigma_oracle(layer)
    scale = np.sqrt(np.outer(np.diag(sig_or), np.diag(sig_or)))
    err = np.max(np.abs(sig_gpu - sig_or) / scale)
    say(f"  max normalized |dSigma| = {err:.3e}")
    assert np.array_equal(sig_gpu, sig_gpu.T)
    assert err <= 1e-6
    s1 = lib.covariance(X[0], alpha=0.5)
    s2 = lib.covariance(X[0], sigma=s1.clone(), alpha=0.25, beta=2.0)
    assert torch.allclose(s2, s1 * 2.5, rtol=1e-12, atol=0)


def test_covariance_streaming_beta(device):
    layer = _layer("spiked_300x333")
    X = x_tensors(layer)[0]
    s1 = lib.covariance(X, alpha=0.5)
    s2 = lib.covariance(X, sigma=s1.clone(), alpha=0.25, beta=2.0)  # 2*(0.5 G) + 0.25 G
    ref = s1 * 2.5
    assert torch.allclose(s2, ref, rtol=1e-12, atol=0)


# ------------------------------------------------------------------ cholesky
@pytest.mark.parametrize("n,kind", [(64, "ar1"), (200, "spd"), (333, "spd"), (1000, "ar1"), (1031, "spd")])
def test_cholesky_parity(device, n, kind):
    say(f"[cholesky] n={n} {kind}")
    rng = np.random.default_rng(n)
    if kind == "ar1":
        idx = np.arange(n)
        sig = 0.9 ** np.abs(idx[:, None] - idx[None, :])
    else:
        g = rng.standard_normal((n, n + 20))
        d = np.exp(rng.standard_normal(n))
        sig = (g @ g.T) / (n + 20) * np.outer(d, d)
    L, info = oracle.cholesky_lower(sig)
    assert info == 0
    A = torch.from_numpy(sig.copy()).to(device)
    A[torch.tril(torch.ones(n, n, dtype=torch.bool, device=device), -1)] = float("nan")  # lower is never read
    U, info_gpu = lib.cholesky(A)
    assert info_gpu == 0
    U = U.cpu().numpy()
    assert np.all(np.tril(U, -1) == 0.0)
    rel = np.linalg.norm(U - L.T) / np.linalg.norm(L)
    back = np.linalg.norm(U.T @ U - sig) / np.linalg.norm(sig)
    say(f"  |U - L^T|/|L| = {rel:.3e}, |U^T U - Sigma|/|Sigma| = {back:.3e}")
    assert back <= 4 * n * 2.2e-16
    assert rel <= 1e-9


@pytest.mark.parametrize("n,bad", [(40, 7), (300, 117), (300, 1)])
def test_cholesky_reports_pivot(device, n, bad):
    say(f"[cholesky-not-pd] n={n} pivot={bad}")
    idx = np.arange(n)
    sig = 0.5 ** np.abs(idx[:, None] - idx[None, :])
    sig[bad - 1, :] = 0.0
    sig[:, bad - 1] = 0.0
    _, info_or = oracle.cholesky_lower(sig)
    with pytest.raises(lib.WsicError) as ei:
        lib.cholesky(torch.from_numpy(sig).to(device))
    assert ei.value.status == lib.E_NOT_PD
    assert ei.value.info == info_or == bad


def test_cholesky_more_panel_workgroups_than_fit(device):
    """n = 20480: a step's panel has 320 workgroups, more than one launch keeps resident, so
    late panel workgroups start after workgroup 0 has finished. The factor must equal the one
    from separate update and panel launches bit for bit and reproduce Sigma on sampled entries
    (regression: the diagonal block was once overwritten in place before all had read it)."""
    n = 20480
    say(f"[cholesky-wide] n={n}")
    g = torch.Generator(device=device).manual_seed(5)
    R = (torch.rand(n, n, generator=g, device=device, dtype=torch.float64) - 0.5) / n
    sig = R + R.T  # off-diagonal row sums below 1: with a unit diagonal, positive definite
    del R
    sig.diagonal().add_(1.0)
    U, _ = lib.cholesky(sig.clone())
    with lib.debug(chol_fused=0):
        U_sep, _ = lib.cholesky(sig.clone())
    assert torch.equal(U, U_sep)
    rng = np.random.default_rng(6)
    I = torch.from_numpy(rng.integers(0, n, 4096)).to(device)
    J = torch.from_numpy(rng.integers(0, n, 4096)).to(device)
    back = ((U[:, I] * U[:, J]).sum(0) - sig[I, J]).abs().max().item()
    say(f"  max |(U^T U - Sigma)_ij| on 4096 entries = {back:.3e}")
    assert back <= 64 * n * 2.0 ** -52


# ------------------------------------------------------------------ SIC pass
def _oracle_factor_on_device(layer):
    L, info = oracle.cholesky_lower(_sigma_oracle(layer))
    assert info == 0
    return L, torch.from_numpy(np.ascontiguousarray(L.T)).to(DEV)


@pytest.mark.parametrize("name", list(LAYERS))
@pytest.mark.parametrize("bits", [1.0, 2.5, 5.0])
def test_sic_codes_parity(device, name, bits):
    layer = _layer(name)
    L, U = _oracle_factor_on_device(layer)
    c = oracle.initial_scale(layer.w, L, bits)
    say(f"[sic] {name} {layer.n_out}x{layer.n_in} c={c:.6g}")
    codes, resid = lib.sic_quantize(w_tensor(layer), U, c, want_resid=True)
    sic = oracle.sic_quantize(layer.w, L, c)
    assert_codes_parity(codes.cpu().numpy(), sic, label=name)
    r = resid.cpu().numpy().astype(np.float64)
    same = np.all(codes.cpu().numpy() == sic["q"], axis=1)
    err = np.abs(r[same] - sic["r"][same]) / sic["alpha"][None, :]
    say(f"  max |dr|/alpha = {err.max():.3e}")
    assert err.max() < 1e-6


def test_sic_identity_factor_is_rtn(device):
    layer = _layer("spiked_300x333")
    n = layer.n_in
    U = torch.eye(n, dtype=torch.float64, device=device)
    c = 0.01
    codes, _ = lib.sic_quantize(w_tensor(layer), U, c)
    ref = np.rint(layer.w.astype(np.float64) / c).astype(np.int64)
    assert np.array_equal(codes.cpu().numpy().astype(np.int64), ref)


def test_sic_strided_inputs(device):
    layer = _layer("blockar1_77x520")
    L, U = _oracle_factor_on_device(layer)
    n_out, n_in = layer.n_out, layer.n_in
    big = torch.zeros((n_out, n_in + 40), dtype=torch.bfloat16, device=device)
    big[:, 7:7 + n_in] = w_tensor(layer)
    Wv = big[:, 7:7 + n_in]
    Ubig = torch.zeros((n_in, n_in + 3), dtype=torch.float64, device=device)
    Ubig[:, :n_in] = U
    codes_big = torch.full((n_out, n_in + 5), -99, dtype=torch.int32, device=device)
    c = oracle.initial_scale(layer.w, L, 2.0)
    lib.sic_quantize(Wv, Ubig[:, :n_in], c, codes=codes_big[:, :n_in])
    sic = oracle.sic_quantize(layer.w, L, c)
    assert_codes_parity(codes_big[:, :n_in].cpu().numpy(), sic, label="strided")
    assert torch.all(codes_big[:, n_in:] == -99)


@pytest.mark.parametrize("which", ["waterfill", "softwater"])
@pytest.mark.parametrize("mode", ["bisect", "secant"])
def test_waterfill_padded_outputs(device, which, mode):
    """Codes and residuals written through row-padded views (ld > n_in): the search must give
    the same c, rate, codes and residuals as with dense outputs, and never write the padding
    (regression: the workspace's second code/residual buffer once took the caller's stride)."""
    layer = _layer("blockar1_77x520")
    L, U = _oracle_factor_on_device(layer)
    n_out, n_in = layer.n_out, layer.n_in
    Wt = w_tensor(layer)
    pad = 37
    codes_big = torch.full((n_out, n_in + pad), -99, dtype=torch.int32, device=device)
    resid_big = torch.full((n_out, n_in + pad), 1234.5, dtype=torch.float32, device=device)
    say(f"[waterfill-padded] {which} {mode} {n_out}x{n_in} ld={n_in + pad}")
    if which == "waterfill":
        run = lambda **kw: lib.waterfill(Wt, U, 2.0, mode=mode, **kw)
    else:
        lam = torch.from_numpy(np.linspace(0.05, 0.25, n_out)).to(device)
        run = lambda **kw: lib.softwater_waterfill(Wt, U, lam, 2.0, mode=mode, **kw)
    dense = run()
    padded = run(codes=codes_big[:, :n_in], resid=resid_big[:, :n_in])
    say(f"  dense c={dense['c']!r} passes={dense['passes']}; padded c={padded['c']!r} passes={padded['passes']}")
    assert padded["c"] == dense["c"] and padded["rate"] == dense["rate"]
    assert torch.equal(codes_big[:, :n_in], dense["codes"])
    assert torch.equal(resid_big[:, :n_in], dense["resid"])
    assert torch.all(codes_big[:, n_in:] == -99)
    assert torch.all(resid_big[:, n_in:] == 1234.5)


@pytest.mark.parametrize("name", ["spiked_200x272", "blockar1_77x520"])
def test_u_lower_triangle_is_not_read(device, name):
    """U's strict lower triangle may hold anything: codes, residuals, the search and both
    distortion modes are unchanged when it is NaN."""
    layer = _layer(name)
    L, U = _oracle_factor_on_device(layer)
    Wt = w_tensor(layer)
    c = oracle.initial_scale(layer.w, L, 2.0)
    Un = U.clone()
    Un[torch.tril(torch.ones_like(Un, dtype=torch.bool), -1)] = float("nan")
    q0, r0 = lib.sic_quantize(Wt, U, c, want_resid=True)
    q1, r1 = lib.sic_quantize(Wt, Un, c, want_resid=True)
    assert torch.equal(q0, q1) and torch.equal(r0, r1)
    wf0 = lib.waterfill(Wt, U, 2.0)
    wf1 = lib.waterfill(Wt, Un, 2.0)
    assert wf0["c"] == wf1["c"] and torch.equal(wf0["codes"], wf1["codes"])
    for mode in ("resid", "direct"):
        D0, _ = lib.distortion(Wt, q0, U, c, resid=r0 if mode == "resid" else None, mode=mode)
        D1, _ = lib.distortion(Wt, q0, Un, c, resid=r0 if mode == "resid" else None, mode=mode)
        assert D0 == D1 and math.isfinite(D1)


# ------------------------------------------------------------------ controller
@pytest.mark.parametrize("name", ["ar1_256_f32", "spiked_300x333", "blockar1_77x520"])
def test_waterfill_bisect_follows_oracle(device, name):
    layer = _layer(name)
    L, U = _oracle_factor_on_device(layer)
    R = 2.0
    say(f"[waterfill-bisect] {name} R={R}")
    wf = lib.waterfill(w_tensor(layer), U, R, mode="bisect")
    ref = oracle.waterfill(layer.w, L, R)
    say(f"  gpu c={wf['c']!r} H={wf['rate']!r} passes={wf['passes']}; oracle c={ref['c']!r} H={ref['rate']!r}")
    assert wf["c"] == pytest.approx(ref["c"], rel=1e-12)
    assert wf["rate"] == pytest.approx(ref["rate"], abs=1e-12)
    assert_codes_parity(wf["codes"].cpu().numpy(), ref["sic"], label=name)


@pytest.mark.parametrize("name", list(LAYERS))
@pytest.mark.parametrize("R", [1.0, 2.0, 3.5])
def test_waterfill_default_parity(device, name, R):
    """The default controller on these small layers meets the rate / c / codes bar."""
    layer = _layer(name)
    L, U = _oracle_factor_on_device(layer)
    say(f"[waterfill-auto] {name} R={R}")
    wf = lib.waterfill(w_tensor(layer), U, R)
    ref = oracle.waterfill(layer.w, L, R)
    say(f"  gpu c={wf['c']:.9g} H={wf['rate']:.7f} passes={wf['passes']}; oracle c={ref['c']:.9g} "
        f"H={ref['rate']:.7f} passes={len(ref['trace'])}")
    assert wf["rate"] <= R
    assert abs(wf["rate"] - ref["rate"]) <= RATE_TOL
    assert abs(wf["c"] / ref["c"] - 1) <= REL_TOL
    # the returned codes are the oracle's codes at the returned grid scale
    sic = oracle.sic_quantize(layer.w, L, wf["c"])
    assert_codes_parity(wf["codes"].cpu().numpy(), sic, label=name)
    assert wf["rate"] == pytest.approx(oracle.entropy_bits(sic["q"]), abs=1e-12)


@pytest.mark.parametrize("name", list(LAYERS))
@pytest.mark.parametrize("R", [1.0, 2.0, 3.5])
def test_waterfill_secant_small_layers(device, name, R):
    """On small layers H(c) moves in visible non-monotone steps, so the fast controller may stop
    at a neighbouring crossing: it must still respect the budget, return the oracle's codes at
    its own c, and sit close to the oracle's c."""
    layer = _layer(name)
    L, U = _oracle_factor_on_device(layer)
    say(f"[waterfill-secant] {name} R={R}")
    wf = lib.waterfill(w_tensor(layer), U, R, mode="secant")
    ref = oracle.waterfill(layer.w, L, R)
    say(f"  gpu c={wf['c']:.9g} H={wf['rate']:.7f} passes={wf['passes']}; oracle c={ref['c']:.9g} "
        f"H={ref['rate']:.7f}")
    assert wf["rate"] <= R
    assert R - wf["rate"] < 2e-3
    assert abs(wf["c"] / ref["c"] - 1) <= 2e-2  # jumps of H here reach 1e-3 bit
    sic = oracle.sic_quantize(layer.w, L, wf["c"])
    assert_codes_parity(wf["codes"].cpu().numpy(), sic, label=name)
    assert wf["rate"] == pytest.approx(oracle.entropy_bits(sic["q"]), abs=1e-12)


# ------------------------------------------------------------------ entropy
@pytest.mark.parametrize("case", ["narrow", "wide", "overflow", "single", "ragged"])
def test_entropy_parity(device, case):
    rng = np.random.default_rng(5)
    if case == "narrow":
        q = np.rint(rng.standard_normal((513, 300)) * 1.3)
    elif case == "wide":
        q = np.rint(rng.standard_normal((200, 1000)) * 500.0)
    elif case == "overflow":
        q = np.rint(rng.standard_t(2, (300, 301)) * 800.0)
        q[0, :5] = [2 ** 31 - 1, -(2 ** 31 - 1), 2048, -2048, 2047]
    elif case == "single":
        q = np.full((64, 64), -3.0)
    else:
        q = np.rint(rng.laplace(0, 3, (7, 5)))
    q = q.astype(np.int32)
    say(f"[entropy] {case} {q.shape}, |q|max={np.abs(q.astype(np.int64)).max()}")
    h, ns = lib.entropy(torch.from_numpy(q).to(device))
    assert h == pytest.approx(oracle.entropy_bits(q), abs=1e-12)
    assert ns == len(np.unique(q))


# ------------------------------------------------------------------ distortion
@pytest.mark.parametrize("name", list(LAYERS))
def test_distortion_parity(device, name):
    layer = _layer(name)
    sig = _sigma_oracle(layer)
    L, U = _oracle_factor_on_device(layer)
    c = oracle.initial_scale(layer.w, L, 2.0)
    say(f"[distortion] {name}")
    Wt = w_tensor(layer)
    codes, resid = lib.sic_quantize(Wt, U, c, want_resid=True)
    q = codes.cpu().numpy().astype(np.int64)
    alpha = oracle.grid_steps(L, c)
    d_or = oracle.distortion_direct(layer.w, q, alpha, sig)
    d_res, w_hat = lib.distortion(Wt, codes, U, c, resid=resid, w_hat_dtype=torch.float32)
    d_dir, _ = lib.distortion(Wt, codes, U, c, mode="direct")
    say(f"  oracle {d_or:.9e}  resid {d_res:.9e}  direct {d_dir:.9e}")
    assert d_res == pytest.approx(d_or, rel=1e-5)
    assert d_dir == pytest.approx(d_or, rel=1e-10)
    np.testing.assert_allclose(w_hat.cpu().numpy(), (q * alpha[None, :]).astype(np.float32), rtol=1e-6)


# ------------------------------------------------------------------ error handling on the device
def test_nonfinite_weight_is_reported(device):
    layer = _layer("spiked_300x333")
    L, U = _oracle_factor_on_device(layer)
    Wt = w_tensor(layer)
    Wt[3, 17] = float("nan")
    with pytest.raises(lib.WsicError) as ei:
        lib.sic_quantize(Wt, U, 0.1)
    assert ei.value.status == lib.E_NONFINITE


@pytest.mark.parametrize("dtype,n_out,n_in,pad", [("bf16", 40, 256, 0), ("bf16", 40, 333, 0),
                                                  ("bf16", 40, 256, 8), ("f32", 24, 260, 0),
                                                  ("f32", 24, 258, 0), ("f32", 24, 256, 4)])
def test_nonfinite_weight_any_position(device, dtype, n_out, n_in, pad):
    """The finiteness check of W reads rows in 16-byte chunks when rows are aligned and element
    by element otherwise (and for a row's tail): a NaN or an Inf anywhere, in either path, is
    reported; a clean layer is not."""
    rng = np.random.default_rng(5)
    full = torch.from_numpy(rng.normal(0, 0.02, (n_out, n_in + pad)).astype(np.float32)).to(device)
    if dtype == "bf16":
        full = full.to(torch.bfloat16)
    W = full[:, :n_in]
    sig = np.eye(n_in)
    U = torch.from_numpy(sig).to(device)
    lib.sic_quantize(W, U, 0.01)  # clean: no error
    if pad:
        full[:, n_in:] = float("nan")  # padding past n_in is not part of the layer
        lib.sic_quantize(W, U, 0.01)
        full[:, n_in:] = 0.0
    for r, j, v in [(0, 0, float("nan")), (1, 9, float("inf")), (n_out // 2, n_in // 2, float("-inf")),
                    (n_out - 1, n_in - 1, float("nan")), (n_out - 2, n_in - 3, float("inf"))]:
        old = W[r, j].item()
        W[r, j] = v
        with pytest.raises(lib.WsicError) as ei:
            lib.sic_quantize(W, U, 0.01)
        assert ei.value.status == lib.E_NONFINITE, (r, j, v)
        W[r, j] = old
    lib.sic_quantize(W, U, 0.01)


def test_nonfinite_activation_is_reported(device):
    layer = _layer("spiked_300x333")
    X = x_tensors(layer)[0]
    X[5, 2] = float("inf")
    with pytest.raises(lib.WsicError) as ei:
        lib.covariance(X)
    assert ei.value.status == lib.E_NONFINITE


def test_code_range_is_reported(device):
    layer = _layer("spiked_300x333")
    L, U = _oracle_factor_on_device(layer)
    with pytest.raises(lib.WsicError) as ei:
        lib.sic_quantize(w_tensor(layer), U, 1e-15)
    assert ei.value.status == lib.E_RANGE


def test_bad_factor_diagonal_is_reported(device):
    layer = _layer("spiked_300x333")
    L, U = _oracle_factor_on_device(layer)
    U[10, 10] = -1.0
    with pytest.raises(lib.WsicError) as ei:
        lib.sic_quantize(w_tensor(layer), U, 0.1)
    assert ei.value.status == lib.E_INVAL


# ------------------------------------------------------------------ interference product variants
@pytest.mark.parametrize("env", [{"fp64_product": 1}, {"guard_scale": 1e300},
                                 {"guard_scale": 3e4}, {"super_blocks": 0},
                                 {"super_blocks": 0, "guard_scale": 3e4}])
@pytest.mark.parametrize("name", ["spiked_300x333", "blockar1_77x520"])
def test_sic_parity_product_variants(device, env, name):
    """fp64 MFMA interference, and the int8 product with every decision re-derived exactly in
    fp64 (error bound forced huge): both must give the oracle's codes."""
    layer = _layer(name)
    L, U = _oracle_factor_on_device(layer)
    c = oracle.initial_scale(layer.w, L, 2.5)
    say(f"[sic-variant] {name} {env}")
    with lib.debug(**env):
        codes, resid = lib.sic_quantize(w_tensor(layer), U, c, want_resid=True)
    sic = oracle.sic_quantize(layer.w, L, c)
    assert_codes_parity(codes.cpu().numpy(), sic, label=f"{name} {env}")


@pytest.mark.parametrize("bits", [7.0, 9.0, 12.0])
def test_sic_parity_large_codes(device, bits):
    """Codes beyond +-127 (the int8 product keeps their excess in per-row lists) and, at the
    highest rate, more of them per row than a list holds (the pass falls back to fp64)."""
    layer = _layer("outliers_130x200")
    L, U = _oracle_factor_on_device(layer)
    c = oracle.initial_scale(layer.w, L, bits)
    codes, _ = lib.sic_quantize(w_tensor(layer), U, c)
    q = codes.cpu().numpy()
    big = (np.abs(q) > 127).sum(axis=1)
    say(f"[sic-large] bits={bits} max|q|={np.abs(q).max()} rows with |q|>127: {(big > 0).sum()}, "
        f"max per row {big.max()}")
    sic = oracle.sic_quantize(layer.w, L, c)
    assert_codes_parity(q, sic, label=f"bits={bits}")
    assert big.max() > 0


def test_entropy_at_the_per_thread_tally_limit(device):
    """A layer large enough that the histogram launch gives each thread its maximum share of
    codes, nearly all of them the same code, so one 8-bit register tally per thread comes close to
    its limit (it must not wrap); the rest at both ends of the tallied range [-7, 7]."""
    n = 512 * 2048 * 250  # more codes than 2048 workgroups of 512 threads cover at 128 per thread
    say(f"[entropy] per-thread limit: {n} codes")
    i = torch.arange(n, device=device, dtype=torch.int64)
    q = torch.where(i % 101 == 0, 7, torch.where(i % 103 == 0, -7, 0)).to(torch.int32).view(-1, 1024)
    del i
    counts = torch.bincount((q.view(-1).to(torch.int64) + 7)).cpu().numpy()
    p = counts[counts > 0].astype(np.float64) / n
    expect = float(-(p * np.log2(p)).sum())
    h, ns = lib.entropy(q)
    say(f"  device {h!r} from counts {expect!r}")
    assert ns == 3
    assert h == pytest.approx(expect, abs=1e-12)
