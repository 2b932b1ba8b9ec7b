"""Device runs of cases whose arithmetic is exact, so the HIP path must reproduce the expected
codes bit for bit with no tie-flip allowance:

  * the hand-worked SIC examples under tests/golden/ (WaterSIC page, Sommario tecnico §2 items
    1-2: reverse-order SIC on the Cholesky factor, steps c/|l_jj|), through wsic_sic_quantize
    and wsic_distortion;
  * exact rounding ties. The pages do not fix a tie rule; the reading taken is round half to
    even (the IEEE default). With Sigma = I the SIC is round-to-nearest per weight, and
    W = (m + 1/2) c (bf16-exact, c a power of two) puts every weight on a tie. With a factor
    whose off-diagonal entries are +-1/2 and weights on a 1/16 grid, every target of the SIC is
    a short binary fraction, so both sides compute it exactly and about a quarter of all
    decisions land exactly on a tie after interference cancellation.
"""
import numpy as np
import pytest
import torch

import oracle
from golden_io import load
from parity import DEV, say
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.lib()
    return torch.device(DEV)


@pytest.mark.parametrize("name", ["hand_sic_2x2.txt", "hand_sic_3x3.txt"])
def test_hand_worked_sic_on_device(device, name):
    g = load(name)
    L = np.atleast_2d(g["L"])
    W = np.atleast_2d(g["W"]).astype(np.float32)
    q_exp = np.atleast_2d(g["q"]).astype(np.int64)
    r_exp = np.atleast_2d(g["r"])
    say(f"[hand] {name}: W {W.shape}, c={g['c']}")
    U = torch.from_numpy(np.ascontiguousarray(L.T)).to(device)
    Wt = torch.from_numpy(W).to(device)
    codes, resid = lib.sic_quantize(Wt, U, float(g["c"]), want_resid=True)
    q = codes.cpu().numpy().astype(np.int64)
    r = resid.cpu().numpy().astype(np.float64)
    say(f"  device q={q.tolist()} r={r.tolist()}")
    assert np.array_equal(q, q_exp)
    assert np.array_equal(r, r_exp)
    for mode in ("resid", "direct"):
        D, w_hat = lib.distortion(Wt, codes, U, float(g["c"]), resid=resid if mode == "resid" else None,
                                  mode=mode, w_hat_dtype=torch.float32)
        say(f"  D ({mode}) = {D!r}, page-worked {g['D']!r}")
        assert D == g["D"]
        assert np.array_equal(w_hat.cpu().numpy(), (q_exp * np.atleast_1d(g["alpha"])[None, :]).astype(np.float32))


def test_identity_factor_ties_round_to_even(device):
    """Sigma = I, W = (m + 1/2) c: every weight sits on a tie; the codes are the even neighbours."""
    rng = np.random.default_rng(11)
    n_out, n_in, c = 96, 333, 2.0 ** -5
    m = rng.integers(-40, 40, size=(n_out, n_in))
    W = ((m + 0.5) * c).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(W)
    assert np.array_equal(workloads.bf16_bits_to_f32(bits), W)  # bf16-exact
    Wt = lib.bf16_from_bits(bits, device)
    U = torch.eye(n_in, dtype=torch.float64, device=device)
    codes, resid = lib.sic_quantize(Wt, U, c, want_resid=True)
    q = codes.cpu().numpy().astype(np.int64)
    expect = np.where(m % 2 == 0, m, m + 1)  # the even one of m, m + 1
    say(f"[ties-identity] {n_out}x{n_in}: all {q.size} weights on a tie, device even: {(q % 2 == 0).mean():.4f}")
    assert np.array_equal(q, expect)
    assert np.all(np.abs(resid.cpu().numpy()) == np.float32(c / 2))


def _dyadic_tie_case(seed, n_out, n_in, density):
    """U = I + strictly upper entries +-1/2 (about `density` per row), c = 1/8, W on a 1/16
    grid (bf16-exact): every SIC target is a multiple of c/4, exactly representable."""
    rng = np.random.default_rng(seed)
    U = np.eye(n_in)
    mask = np.triu(rng.random((n_in, n_in)) < density / n_in, 1)
    U[mask] = rng.choice([-0.5, 0.5], size=int(mask.sum()))
    c = 0.125
    W = (rng.integers(-12, 13, size=(n_out, n_in)) / 16.0).astype(np.float32)
    return U, c, W


@pytest.mark.parametrize("variant", [{}, {"fp64_product": 1}, {"super_blocks": 0}])
def test_ties_after_interference_round_to_even(device, variant):
    n_out, n_in = 200, 700
    U, c, W = _dyadic_tie_case(3, n_out, n_in, density=3.0)
    L = U.T
    sic = oracle.sic_quantize(W, L, c)
    z = sic["t"] / sic["alpha"][None, :]
    ties = (z - np.floor(z)) == 0.5
    say(f"[ties-interference] {n_out}x{n_in} {variant}: {int(ties.sum())} exact ties "
        f"({ties.mean():.3f} of decisions), |q|max={np.abs(sic['q']).max()}")
    assert ties.sum() > 0.15 * ties.size
    assert np.all(sic["q"][ties] % 2 == 0)  # the oracle rounds ties to even
    bits = workloads.f32_to_bf16_bits(W)
    assert np.array_equal(workloads.bf16_bits_to_f32(bits), W)
    Wt = lib.bf16_from_bits(bits, device)
    Ut = torch.from_numpy(U).to(device)
    with lib.debug(**variant):
        codes, resid = lib.sic_quantize(Wt, Ut, c, want_resid=True)
    q = codes.cpu().numpy().astype(np.int64)
    n_diff_rows = int(np.any(q != sic["q"], axis=1).sum())
    say(f"  device: rows differing {n_diff_rows}/{n_out}")
    assert np.array_equal(q, sic["q"])
    assert np.array_equal(resid.cpu().numpy().astype(np.float64), sic["r"])
