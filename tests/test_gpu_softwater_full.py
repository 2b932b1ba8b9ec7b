"""SoftWater parity on the LM-head workload at full size (32000 classes x 4096 inputs, 8192
calibration rows), in the launch configuration the benchmark times (``bench.py --softwater``):

  * class curvatures of all 8192 rows against the fp64 oracle, within the bound of fp32
    summation of the logits (derived in tests/test_gpu_softwater.py);
  * class-aware waterfilling at 1.5 and 3 bits: codes, residuals and per-row KL distortion of
    sampled classes against the oracle's SIC at the device's c and curvatures (rows are
    independent given U, c and lambda_k);
  * the rate equals the oracle's entropy of all codes and sits inside the budget; the streaming
    KL estimate equals the sum of its per-row terms.
"""
import numpy as np
import pytest
import torch

from oracle import softwater as sw
from oracle import watersic as ws
from parity import RATE_TOL, assert_codes_parity, say, w_tensor, x_tensors
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(1200)]

NAME = "lmhead_32000x4096"
SMOOTHING = 0.05
N_SAMPLE_ROWS = 12
_state = {}


def _setup():
    if _state:
        return _state
    say(f"[softwater-full] generating {NAME}")
    layer = workloads.named_workload(NAME)
    Wt = w_tensor(layer)
    X = x_tensors(layer)
    say("[softwater-full] covariance, cholesky, class curvatures")
    sigma = lib.covariance_chunks(X)
    U, _ = lib.cholesky(sigma.clone())
    lam = lib.softmax_curvature_chunks(X, Wt, SMOOTHING)
    torch.cuda.synchronize()
    _state.update(layer=layer, Wt=Wt, sigma=sigma, U=U, lam=lam)
    return _state


def test_curvature_full():
    st = _setup()
    layer = st["layer"]
    lam = st["lam"].cpu().numpy()
    say("[softwater-full] oracle curvatures over all calibration rows (fp64)")
    xs = [np.asarray(c, dtype=np.float64) for c in layer.x_chunks]
    ref = sw.softmax_curvature(xs, layer.w, SMOOTHING)
    # the largest sum_i |x_i w_ki| over calibration rows and classes
    Wabs = np.abs(layer.w.astype(np.float64)).T
    worst = max(float((np.abs(X[r0:r0 + 512]) @ Wabs).max()) for X in xs for r0 in range(0, X.shape[0], 512))
    tol = 4.0 * (layer.n_in + 1) * 2.0 ** -24 * worst + 2.0 ** -20
    rel = np.abs(lam / ref - 1.0)
    say(f"  lambda: max rel error {rel.max():.3e} (bound {tol:.3e}), range [{lam.min():.3e}, {lam.max():.3e}]")
    assert rel.max() <= tol


@pytest.mark.parametrize("R", [1.5, 3.0])
def test_softwater_full(R):
    st = _setup()
    layer, Wt, U, lam_t = st["layer"], st["Wt"], st["U"], st["lam"]
    say(f"[softwater-full] R={R}: class-aware waterfill, entropy, KL distortion")
    wf = lib.softwater_waterfill(Wt, U, lam_t, R)
    codes, resid, c = wf["codes"], wf["resid"], wf["c"]
    h, nsym = lib.entropy(codes)
    D, _ = lib.softwater_distortion(codes, U, c, lam_t, resid)
    say(f"  c={c:.9g} rate={wf['rate']:.7f} passes={wf['passes']} D_KL={D:.6e} symbols={nsym}")

    lam = lam_t.cpu().numpy()
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, layer.n_out - 1],
                                     rng.choice(layer.n_out, N_SAMPLE_ROWS - 2, replace=False)]))
    U_host = U.cpu().numpy()
    L = U_host.T
    say(f"  oracle class-aware SIC on {len(rows)} classes")
    sic = sw.sic_quantize(layer.w[rows], L, lam[rows], c)
    rows_t = torch.from_numpy(rows).cuda()
    assert_codes_parity(codes[rows_t].cpu().numpy(), sic, label=f"{NAME} softwater R={R} sample")
    s = np.sqrt(lam[rows])[:, None]
    r_s = resid[rows_t].cpu().numpy().astype(np.float64)
    assert (np.abs(r_s / s - sic["r"]) / sic["alpha"]).max() < 1e-6
    # per-row KL terms: 1/2 sum_j U_jj^2 r'_kj^2 against 1/2 lambda_k e_k Sigma e_k^T
    d2 = np.diag(U_host) ** 2
    E = layer.w[rows].astype(np.float64) - sic["q"] * sic["alpha"]
    sigma_host = st["sigma"].cpu().numpy()
    kl_or = 0.5 * lam[rows] * np.einsum("ij,ij->i", E @ sigma_host, E)
    del sigma_host
    kl_dev = 0.5 * (d2[None, :] * r_s ** 2).sum(axis=1)
    np.testing.assert_allclose(kl_dev, kl_or, rtol=1e-5)
    # the streaming estimate is the sum of the per-row terms of all rows
    r_all = resid.double()
    D_sum = 0.5 * float((r_all * r_all * torch.diagonal(U).pow(2)[None, :]).sum())
    assert D == pytest.approx(D_sum, rel=1e-9)

    say("  oracle entropy of the pooled codes")
    h_or = ws.entropy_bits(codes.cpu().numpy())
    assert h == pytest.approx(h_or, abs=1e-12)
    assert wf["rate"] == pytest.approx(h_or, abs=1e-12)
    assert wf["rate"] <= R and R - wf["rate"] < RATE_TOL
