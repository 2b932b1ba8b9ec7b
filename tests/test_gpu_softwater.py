"""GPU parity of the SoftWater path (class curvatures, class-aware waterfilling, KL distortion)
against the fp64 oracle (oracle/softwater.py), through the C ABI.

Curvature tolerance. On the bf16 MFMA path each logit l = sum_i x_i w_i is summed in fp32: its
error is at most n * 2^-24 * sum_i |x_i w_i| (n terms, each product exact). A logit error d moves
p_k by at most a factor exp(2 |d|max) (numerator and normalizer), so p~(1 - p~) and its mean by
a relative 4 |d|max to first order; the test allows the largest such bound over the
calibration rows and classes. Every path also rounds each logit to fp32 (|d| <= 2^-24 |l| <=
2^-24 sum_i |x_i w_i|) and evaluates exp in fp32 (2^-20 relative allowance).

Codes, c and the rate are graded as for WaterSIC (tests/parity.py) with both sides on the same
class curvatures (the device's), so the grids are identical."""
import numpy as np
import pytest
import torch

from oracle import softwater as sw
from oracle import watersic as ws
from parity import DEV, RATE_TOL, REL_TOL, assert_codes_parity, say, w_tensor, x_tensors
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu

HEADS = {
    # name: (n_classes, n_in, calibration rows, kwargs) -- the LM-head recipe at test size
    "head_96x200": (96, 200, 600, dict(dtype="bf16", rank=16)),
    "head_300x256": (300, 256, 640, dict(dtype="bf16", rank=16)),
    "head_64x136_f32": (64, 136, 300, dict(dtype="f32", rank=8)),
}


def _head(name, seed=0):
    K, n, rows, kw = HEADS[name]
    return workloads.make_layer("lmhead", K, n, rows, seed=seed, name=name, **kw)


@pytest.fixture(scope="module")
def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.lib()
    return torch.device(DEV)


def _curv_tol(layer, x_chunks64, fp32_sums):
    W = np.abs(layer.w.astype(np.float64))
    n = W.shape[1]
    worst = 0.0
    for X in x_chunks64:
        worst = max(worst, float((np.abs(X) @ W.T).max()))
    return 4.0 * ((n if fp32_sums else 0) + 1) * 2.0 ** -24 * worst + 2.0 ** -20


@pytest.mark.parametrize("name", list(HEADS))
@pytest.mark.parametrize("eps", [0.0, 0.05])
def test_curvature_parity(device, name, eps):
    layer = _head(name)
    xs = [np.asarray(c, dtype=np.float64) for c in layer.x_chunks]
    ref = sw.softmax_curvature(xs, layer.w, eps)
    mfma = layer.dtype == "bf16"
    for generic in ([False, True] if mfma else [False]):
        with lib.debug(logits_generic=1 if generic else 0):
            lam = lib.softmax_curvature_chunks(x_tensors(layer), w_tensor(layer), eps).cpu().numpy()
        tol = _curv_tol(layer, xs, mfma and not generic)
        rel = np.abs(lam / ref - 1.0)
        say(f"[curvature] {name} eps={eps} generic={generic}: max rel {rel.max():.3e} (tol {tol:.3e})")
        assert rel.max() <= tol


def test_curvature_streaming_beta(device):
    """lambda <- beta lambda + alpha (...): two calls over halves equal one call over all rows."""
    layer = _head("head_96x200")
    X = x_tensors(layer)
    Xall = torch.cat(X, 0)
    W = w_tensor(layer)
    one = lib.softmax_curvature(Xall, W, 0.02)
    h = Xall.shape[0] // 2 + 5
    lam = lib.softmax_curvature(Xall[:h], W, 0.02, alpha=1.0 / Xall.shape[0])
    lam = lib.softmax_curvature(Xall[h:], W, 0.02, lam=lam, alpha=1.0 / Xall.shape[0], beta=1.0)
    np.testing.assert_allclose(lam.cpu().numpy(), one.cpu().numpy(), rtol=1e-12)


def test_curvature_rejects_bad_smoothing(device):
    layer = _head("head_96x200")
    with pytest.raises(lib.WsicError):
        lib.softmax_curvature(x_tensors(layer)[0], w_tensor(layer), 1.5)


def _factor(layer):
    L, info = ws.cholesky_lower(ws.covariance([np.asarray(c, dtype=np.float64) for c in layer.x_chunks]))
    assert info == 0
    return L, torch.from_numpy(np.ascontiguousarray(L.T)).to(DEV)


@pytest.mark.parametrize("name", ["head_96x200", "head_300x256", "head_64x136_f32"])
@pytest.mark.parametrize("R", [1.5, 3.0])
def test_softwater_waterfill_parity(device, name, R):
    layer = _head(name)
    L, U = _factor(layer)
    lam_t = lib.softmax_curvature_chunks(x_tensors(layer), w_tensor(layer), 0.05)
    lam = lam_t.cpu().numpy()
    wf = lib.softwater_waterfill(w_tensor(layer), U, lam_t, R, mode="bisect")
    ref = sw.waterfill(layer.w, L, lam, R)
    say(f"[softwater] {name} R={R}: gpu c={wf['c']:.12g} H={wf['rate']:.7f} passes={wf['passes']}; "
        f"oracle c={ref['c']:.12g} H={ref['rate']:.7f}")
    # the bisection replays the oracle's search on the same grids
    assert wf["c"] == pytest.approx(ref["c"], rel=1e-12)
    sic = sw.sic_quantize(layer.w, L, lam, wf["c"])
    q = wf["codes"].cpu().numpy()
    assert_codes_parity(q, sic, label=name)
    assert wf["rate"] == pytest.approx(ws.entropy_bits(q), abs=1e-12)
    assert wf["rate"] <= R and abs(wf["rate"] - ref["rate"]) <= RATE_TOL
    # residuals are those of the rescaled rows
    same = np.all(q == sic["q"], axis=1)
    s = np.sqrt(lam)[:, None]
    r = wf["resid"].cpu().numpy().astype(np.float64) / s
    err = np.abs(r[same] - sic["r"][same]) / sic["alpha"][same]
    say(f"  max |dr|/alpha = {err.max():.3e}")
    assert err.max() < 1e-6
    # KL distortion: streaming estimate vs the definition (Sigma from the calibration rows)
    D, w_hat = lib.softwater_distortion(wf["codes"], U, wf["c"], lam_t, wf["resid"], w_hat_dtype=torch.float32)
    sigma = L @ L.T
    D_def = sw.kl_distortion(layer.w, sic["q"], sic["alpha"], sigma, lam)
    say(f"  D_KL gpu {D:.6e} oracle {D_def:.6e}")
    assert D == pytest.approx(D_def, rel=REL_TOL)
    wh_ref = (sic["q"] * sic["alpha"]).astype(np.float32)
    np.testing.assert_allclose(w_hat.cpu().numpy()[same], wh_ref[same], rtol=1e-6, atol=0)


def test_softwater_unit_curvature_is_watersic(device):
    """lambda = 1 everywhere: the class-aware path is WaterSIC itself."""
    layer = _head("head_96x200")
    _, U = _factor(layer)
    W = w_tensor(layer)
    ones = torch.ones(layer.n_out, dtype=torch.float64, device=DEV)
    a = lib.softwater_waterfill(W, U, ones, 2.0, mode="bisect")
    b = lib.waterfill(W, U, 2.0, mode="bisect")
    assert a["c"] == b["c"] and a["rate"] == b["rate"]
    assert torch.equal(a["codes"], b["codes"])


@pytest.mark.parametrize("bad", [0.0, -1.0, float("nan"), float("inf")])
def test_softwater_rejects_bad_curvature(device, bad):
    layer = _head("head_96x200")
    _, U = _factor(layer)
    lam = torch.full((layer.n_out,), 0.01, dtype=torch.float64, device=DEV)
    lam[7] = bad
    with pytest.raises(lib.WsicError) as e:
        lib.softwater_waterfill(w_tensor(layer), U, lam, 2.0)
    assert e.value.status == lib.E_INVAL
