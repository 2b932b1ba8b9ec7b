"""GPU parity of the practical corrections of the WaterSIC page, §2 item 4, through the C ABI:
the per-row LMMSE factors against the oracle's definition (Sigma = L L^T of the same factor), and
dead-feature removal (live columns, gathers, codes scattered back) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import DEV, assert_codes_parity, say, w_tensor
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.lib()
    return torch.device(DEV)


@pytest.mark.parametrize("R", [1.0, 3.0])
def test_lmmse_scale_parity(device, R):
    layer = workloads.make_layer("spiked", 300, 333, 900, seed=0, name="spiked_300x333", dtype="bf16", rank=16)
    L, info = oracle.cholesky_lower(oracle.covariance(layer.x_chunks))
    U = torch.from_numpy(np.ascontiguousarray(L.T)).to(DEV)
    Wt = w_tensor(layer)
    wf = lib.waterfill(Wt, U, R)
    gamma, d_before, d_after = lib.lmmse_scale(Wt, U, wf["resid"])
    sic = oracle.sic_quantize(layer.w, L, wf["c"])
    q = wf["codes"].cpu().numpy()
    assert_codes_parity(q, sic, label="lmmse layer")
    W_hat = q * sic["alpha"][None, :]
    ref = oracle.lmmse_scale(layer.w, W_hat, L @ L.T)
    g = gamma.cpu().numpy()
    say(f"[lmmse] R={R}: gamma in [{g.min():.6f}, {g.max():.6f}], D {d_before:.6e} -> {d_after:.6e} "
        f"(oracle {ref['D_before']:.6e} -> {ref['D_after']:.6e})")
    # the residuals are fp32: their rounding (2^-24 relative) bounds the factors' error
    np.testing.assert_allclose(g, ref["gamma"], rtol=0, atol=1e-6)
    assert d_before == pytest.approx(ref["D_before"], rel=1e-5)
    assert d_after == pytest.approx(ref["D_after"], rel=1e-5)
    assert d_after <= d_before
    D_dev, _ = lib.distortion(Wt, wf["codes"], U, wf["c"], resid=wf["resid"])
    assert d_before == pytest.approx(D_dev, rel=1e-9)


def test_dead_feature_removal(device):
    rng = np.random.default_rng(4)
    n_out, n_in, rows = 120, 150, 700
    X = rng.standard_normal((rows, n_in)) * np.exp(0.5 * rng.standard_normal(n_in))[None, :]
    dead = [0, 17, 63, 64, 149]
    X[:, dead] = 0.0
    X[:, 90] *= 1e-9  # near-zero variance: below tau * max
    Xf = X.astype(np.float32)
    W = (rng.standard_normal((n_out, n_in)) * 0.02).astype(np.float32)
    Xt, Wt = torch.from_numpy(Xf).to(DEV), torch.from_numpy(W).to(DEV)
    sigma = lib.covariance(Xt, alpha=1.0 / rows)
    with pytest.raises(lib.WsicError):
        lib.cholesky(sigma.clone())
    tau = 1e-12
    idx, pos, n_live = lib.live_features(sigma, tau)
    sig_h = sigma.cpu().numpy()
    live = oracle.live_features(sig_h, tau)
    say(f"[dead] {n_in - n_live} dead columns: {sorted(set(range(n_in)) - set(live.tolist()))}")
    assert n_live == len(live) == n_in - len(dead) - 1
    np.testing.assert_array_equal(idx[:n_live].cpu().numpy(), live)
    p = pos.cpu().numpy()
    np.testing.assert_array_equal(p[live], np.arange(n_live))
    assert np.all(p[np.setdiff1d(np.arange(n_in), live)] == -1)
    W_l, S_l = lib.gather_features(Wt, idx, n_live, sigma)
    np.testing.assert_array_equal(W_l.cpu().numpy(), W[:, live])
    np.testing.assert_array_equal(S_l.cpu().numpy(), sig_h[np.ix_(live, live)])
    U_l, _ = lib.cholesky(S_l.clone())
    wf = lib.waterfill(W_l, U_l, 2.0)
    q_full = lib.scatter_codes(wf["codes"], pos, n_in).cpu().numpy()
    assert np.all(q_full[:, np.setdiff1d(np.arange(n_in), live)] == 0)
    np.testing.assert_array_equal(q_full[:, live], wf["codes"].cpu().numpy())
    # the live problem against the oracle at the device's factor and scale
    Ul_h = U_l.cpu().numpy()
    sic = oracle.sic_quantize(W[:, live].astype(np.float64), Ul_h.T, wf["c"])
    assert_codes_parity(wf["codes"].cpu().numpy(), sic, label="live layer")
    # dead columns add nothing to the distortion of the full layer beyond their own (tiny) variance
    W_hat = np.zeros((n_out, n_in))
    W_hat[:, live] = q_full[:, live] * sic["alpha"][None, :]
    d_full = oracle.distortion_direct(W, W_hat, np.ones(n_in), sig_h)
    d_live = oracle.distortion_from_residuals(sic["r"], Ul_h.T)
    assert d_full == pytest.approx(d_live, rel=1e-6)
