"""GPU parity of the per-column rate and of the Gaussian limit report (WaterSIC page, §3 Limiti
teorici), through the C ABI: the mean column entropy exactly against the oracle (register tallies,
LDS window and overflow list all exercised), the controller holding that rate (bisection replays
the oracle's search), and the high-rate Gaussian limit against the oracle's reverse waterfilling
over the eigenvalues of Sigma, with the measured gap of WaterSIC against 1/2 log2(2 pi e / 12)."""
import numpy as np
import pytest
import torch

import oracle
from parity import DEV, RATE_TOL, assert_codes_parity, say, w_tensor, x_tensors
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.lib()
    return torch.device(DEV)


@pytest.mark.parametrize("shape,spread", [((700, 45), 3), ((1030, 77), 40), ((513, 33), 400), ((64, 8), 2)])
def test_entropy_columns_parity(device, shape, spread):
    rng = np.random.default_rng(spread)
    q = np.rint(rng.standard_normal(shape) * spread * rng.uniform(0.2, 1.5, size=shape[1])[None, :])
    q[0, 0] = 2 ** 31 - 1
    q[-1, -1] = -(2 ** 31) + 1
    q = q.astype(np.int32)
    h = lib.entropy_columns(torch.from_numpy(q).to(DEV))
    ref = oracle.entropy_bits_columns(q)
    say(f"[colrate] {shape} spread {spread}: device {h:.12f} oracle {ref:.12f}")
    assert h == pytest.approx(ref, abs=1e-12)
    hp, _ = lib.entropy(torch.from_numpy(q).to(DEV))
    assert hp >= h - 1e-12


def test_entropy_columns_strided(device):
    rng = np.random.default_rng(1)
    big = torch.from_numpy(rng.integers(-9, 10, size=(300, 200)).astype(np.int32)).to(DEV)
    view = big[:, 13:170]
    assert lib.entropy_columns(view) == pytest.approx(oracle.entropy_bits_columns(view.cpu().numpy()), abs=1e-12)


def _layer():
    return workloads.make_layer("spiked", 300, 333, 900, seed=0, name="spiked_300x333", dtype="bf16", rank=16)


@pytest.mark.parametrize("R", [2.0, 4.0])
def test_waterfill_columns_mode_follows_oracle(device, R):
    layer = _layer()
    L, info = oracle.cholesky_lower(oracle.covariance(layer.x_chunks))
    U = torch.from_numpy(np.ascontiguousarray(L.T)).to(DEV)
    wf = lib.waterfill(w_tensor(layer), U, R, mode="bisect", rate_mode="columns")
    ref = oracle.waterfill(layer.w, L, R, rate_fn=oracle.entropy_bits_columns)
    say(f"[colrate] R={R}: gpu c={wf['c']:.12g} H={wf['rate']:.7f}; oracle c={ref['c']:.12g} H={ref['rate']:.7f}")
    assert wf["c"] == pytest.approx(ref["c"], rel=1e-12)
    q = wf["codes"].cpu().numpy()
    assert_codes_parity(q, oracle.sic_quantize(layer.w, L, wf["c"]), label="columns mode")
    assert wf["rate"] == pytest.approx(oracle.entropy_bits_columns(q), abs=1e-12)
    assert wf["rate"] <= R and abs(wf["rate"] - ref["rate"]) <= RATE_TOL
    # the default controller reaches the same target on the per-column rate
    wd = lib.waterfill(w_tensor(layer), U, R, rate_mode="columns", mode="secant")
    assert wd["rate"] <= R and R - wd["rate"] < 2e-3


def test_gap_to_gaussian_limit(device):
    """Gaussian rows (16384 x 48, f32), AR(1) inputs: the per-column rate of WaterSIC at about 5
    bits sits 0.2546 bit (+-0.03) above the Gaussian limit at its distortion; the device's
    high-rate limit equals the oracle's reverse waterfilling, whose water level lies below every
    eigenvalue here."""
    rng = np.random.default_rng(7)
    n_out, n_in, rows = 16384, 48, 4000
    sd = 0.02
    W = (rng.standard_normal((n_out, n_in)) * sd).astype(np.float32)
    x = np.empty((rows, n_in))
    x[:, 0] = rng.standard_normal(rows)
    for i in range(1, n_in):
        x[:, i] = 0.8 * x[:, i - 1] + 0.6 * rng.standard_normal(rows)
    X = x.astype(np.float32)
    Wt, Xt = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
    sigma = lib.covariance(Xt, alpha=1.0 / rows)
    U, _ = lib.cholesky(sigma.clone())
    R = 5.0
    wf = lib.waterfill(Wt, U, R, rate_mode="columns")
    D, _ = lib.distortion(Wt, wf["codes"], U, wf["c"], resid=wf["resid"])
    rg, var = lib.gaussian_rate(Wt, U, D)
    # oracle: exact reverse waterfilling on Sigma's eigenvalues and the weight variance
    sig_h = sigma.cpu().numpy()
    mu = np.linalg.eigvalsh(sig_h)
    var_or = float(np.mean(W.astype(np.float64) ** 2))
    theta = D / W.size
    assert var == pytest.approx(var_or, rel=1e-12)
    assert theta < var_or * mu.min()  # the high-rate form is exact here
    rg_or = oracle.gaussian_rate(mu, var_or, theta)
    rg_hi = oracle.gaussian_rate_high(np.diag(U.cpu().numpy()), var_or, theta)
    say(f"[gap] rate {wf['rate']:.5f}  gaussian {rg:.5f} (oracle {rg_or:.5f})  gap {wf['rate'] - rg:.4f}")
    assert rg == pytest.approx(rg_hi, abs=1e-12)
    assert rg == pytest.approx(rg_or, abs=1e-8)
    assert wf["rate"] - rg == pytest.approx(oracle.RATE_GAP_BITS, abs=0.03)
