"""wsic_distortion_noalloc, the entry point for callers that cannot allocate: through the C ABI
it must return what wsic_distortion returns on the same inputs, on consecutive calls that share
the static scratch (the second on a smaller layer, so stale partials of the first would show),
in both distortion modes, with the dequantized weights; and it must allocate nothing."""
import gc

import numpy as np
import pytest
import torch

import oracle
from parity import DEV, say, w_tensor
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu


def _case(recipe, n_out, n_in, rows, seed, **kw):
    layer = workloads.make_layer(recipe, n_out, n_in, rows, seed=seed, **kw)
    L, info = oracle.cholesky_lower(oracle.covariance(layer.x_chunks))
    assert info == 0
    U = torch.from_numpy(np.ascontiguousarray(L.T)).to(DEV)
    Wt = w_tensor(layer)
    c = oracle.initial_scale(layer.w, L, 2.0)
    codes, resid = lib.sic_quantize(Wt, U, c, want_resid=True)
    return Wt, U, c, codes, resid


def test_noalloc_distortion_equals_workspace_call():
    assert torch.cuda.is_available()
    cases = [("spiked", 300, 333, 900, 0, dict(dtype="bf16", rank=16)),   # larger first
             ("ar1", 77, 200, 500, 1, dict(dtype="f32", rho=0.9))]         # then smaller
    for recipe, n_out, n_in, rows, seed, kw in cases:
        Wt, U, c, codes, resid = _case(recipe, n_out, n_in, rows, seed, **kw)
        for mode in ("resid", "direct"):
            d_ws, wh_ws = lib.distortion(Wt, codes, U, c, resid=resid if mode == "resid" else None, mode=mode,
                                         w_hat_dtype=torch.float32)
            wh = torch.full((n_out, n_in), float("nan"), dtype=torch.float32, device=DEV)
            # the garbage collector must not free tensors of earlier tests inside the measured
            # call (a drop of the count is no allocation, but it would hide one)
            gc.collect()
            gc.disable()
            try:
                torch.cuda.synchronize()
                before = torch.cuda.memory_allocated()
                d_na = lib.distortion_noalloc(Wt, codes, U, c, resid=resid if mode == "resid" else None,
                                              mode=mode, w_hat=wh)
                torch.cuda.synchronize()
                after = torch.cuda.memory_allocated()
            finally:
                gc.enable()
            assert after == before
            say(f"[noalloc] {recipe} {n_out}x{n_in} {mode}: workspace call {d_ws!r}, static scratch {d_na!r}")
            assert d_na == d_ws
            assert torch.equal(wh, wh_ws)


def test_noalloc_rejects_layers_beyond_its_scratch():
    Wt, U, c, codes, resid = _case("ar1", 8, 64, 200, 2, dtype="f32", rho=0.5)
    st = lib.lib().wsic_distortion_noalloc(
        lib._p(Wt.data_ptr()), lib.F32, 1 << 20, 32768, 32768, lib._p(codes.data_ptr()), 32768,
        lib._p(U.data_ptr()), 32768, c, lib._p(resid.data_ptr()), 32768, lib.D_RESID,
        lib.ctypes.byref(lib._d(0)), None, lib.F32, 32768, None)
    assert st == lib.E_WORKSPACE
    assert b"static" in lib.lib().wsic_last_error()
