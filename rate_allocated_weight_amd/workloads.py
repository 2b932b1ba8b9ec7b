"""Seeded synthetic layer workloads: a weight matrix W and calibration activations X.

This module only draws inputs. It holds none of the quantizer's arithmetic, and both the
fp64 oracle (tests) and the HIP path (tests, bench) read the arrays it returns.

Recipes (one per named workload; every shape and distribution is a parameter so that tests
can draw the same structure at small, ragged sizes):

* ``ar1``     W ~ N(0, w_std^2). X rows follow an AR(1) recursion along the feature axis,
              x_0 = z_0, x_i = rho*x_{i-1} + sqrt(1-rho^2)*z_i, so Sigma_ij = rho^|i-j|.
              Optional per-channel log-normal scales s_i = exp(N(0, scale_sigma^2)) give
              Sigma = diag(s) R diag(s). Optional whole-column outliers in W.
* ``spiked``  Sigma = V diag(lambda) V^T + diag(d) with V the Q factor of a Gaussian
              n_in x rank matrix, lambda_k = 10^U(1,3), d_i = exp(N(0,1)).
              X = Z_a diag(sqrt(lambda)) V^T + Z_b diag(sqrt(d)). W Student-t (nu) scaled to
              a target std, or Gaussian.
* ``lmhead``  W row i has width sigma_i proportional to p_i^(-1/4) with Zipf class
              frequencies p_i ~ (i+1)^(-s), normalised to a target RMS; X from ``spiked``.
* ``blockar1`` Sigma = D blockdiag(AR(1) blocks) D with D = diag(exp(N(0,1))), X streamed
              in row chunks, the AR(1) recursion restarted at every block edge.

Floating point: everything is drawn in float64, rounded to float32 (round to nearest even),
and for bf16 workloads rounded again to bfloat16 (round to nearest even on the float32 bit
pattern). bf16 arrays are returned as ``uint16`` bit patterns plus their exact float32
values, so both sides see identical numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator, List, Optional, Sequence

import numpy as np

__all__ = [
    "Layer",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_layer",
    "named_workload",
    "NAMED",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16 rounding of non-finite values is not supported")
    # finite values: u + 0x8000 stays below 2^32, so 32-bit arithmetic is exact
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Layer:
    """One synthetic layer. ``w`` / ``x_chunks`` hold the exact float32 values; for bf16
    workloads ``w_bits`` / ``x_bits_chunks`` hold the uint16 patterns the device reads."""

    name: str
    dtype: str  # "f32" or "bf16"
    w: np.ndarray  # (n_out, n_in) float32
    x_chunks: List[np.ndarray]  # each (rows, n_in) float32
    targets: List[float]
    w_bits: Optional[np.ndarray] = None
    x_bits_chunks: Optional[List[np.ndarray]] = None

    @property
    def n_out(self) -> int:
        return self.w.shape[0]

    @property
    def n_in(self) -> int:
        return self.w.shape[1]

    @property
    def n_rows(self) -> int:
        return sum(c.shape[0] for c in self.x_chunks)


def _finish(name, dtype, w64, x64_chunks, targets) -> Layer:
    w32 = w64.astype(np.float32)
    xs32 = [c.astype(np.float32) for c in x64_chunks]
    if dtype == "f32":
        return Layer(name, dtype, np.ascontiguousarray(w32), [np.ascontiguousarray(c) for c in xs32],
                     list(targets))
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    wb = f32_to_bf16_bits(w32)
    xbs = [f32_to_bf16_bits(c) for c in xs32]
    return Layer(name, dtype, bf16_bits_to_f32(wb), [bf16_bits_to_f32(b) for b in xbs], list(targets),
                 w_bits=wb, x_bits_chunks=xbs)


def _student_t(rng: np.random.Generator, nu: float, shape, std: float) -> np.ndarray:
    # Student-t with nu > 2 has variance nu/(nu-2); rescale to the requested std.
    return rng.standard_t(nu, size=shape) * (std / math.sqrt(nu / (nu - 2.0)))


def _ar1_rows(rng: np.random.Generator, rows: int, n: int, rho: float, block: int = 0) -> np.ndarray:
    """AR(1) along the feature axis; restarted every ``block`` features when block > 0.

    x_0 = z_0, x_i = rho x_{i-1} + a z_i (a = sqrt(1 - rho^2)), evaluated in that order by a
    first-order recursive filter (scipy's lfilter: per element the products a z_i and
    rho x_{i-1} and their sum, as written)."""
    from scipy.signal import lfilter

    z = rng.standard_normal((rows, n))
    a = math.sqrt(1.0 - rho * rho)
    if block <= 0:
        block = n
    x = np.empty_like(z)
    for s0 in range(0, n, block):
        s1 = min(n, s0 + block)
        x[:, s0] = z[:, s0]
        if s1 - s0 > 1:
            x[:, s0 + 1:s1] = lfilter([a], [1.0, -rho], z[:, s0 + 1:s1], axis=-1,
                                      zi=rho * z[:, s0:s0 + 1])[0]
    return x


def _spiked_factors(rng: np.random.Generator, n_in: int, rank: int):
    g = rng.standard_normal((n_in, rank))
    v, _ = np.linalg.qr(g)
    lam = 10.0 ** rng.uniform(1.0, 3.0, size=rank)
    d = np.exp(rng.standard_normal(n_in))
    return v, lam, d


_RECIPE_IDS = {"ar1": 1, "spiked": 2, "lmhead": 3, "blockar1": 4}


def make_layer(recipe: str, n_out: int, n_in: int, n_rows: int, *, seed: int = 0, dtype: str = "bf16",
               targets: Sequence[float] = (2.0,), chunk_rows: int = 0, name: Optional[str] = None,
               **kw) -> Layer:
    """Draw one layer following ``recipe`` (see module docstring) at the given shape."""
    if recipe not in _RECIPE_IDS:
        raise ValueError(f"unknown recipe {recipe!r}")
    ss = np.random.SeedSequence([int(seed), _RECIPE_IDS[recipe]])
    n_chunks = 1 if chunk_rows <= 0 else -(-n_rows // chunk_rows)
    kids = ss.spawn(2 + n_chunks)
    rw = np.random.Generator(np.random.PCG64(kids[0]))
    rs = np.random.Generator(np.random.PCG64(kids[1]))
    chunk_rngs = [np.random.Generator(np.random.PCG64(k)) for k in kids[2:]]
    chunk_sizes = [n_rows] if chunk_rows <= 0 else [min(chunk_rows, n_rows - i * chunk_rows)
                                                   for i in range(n_chunks)]
    name = name or f"{recipe}_{n_out}x{n_in}"

    if recipe == "ar1":
        w_std = kw.get("w_std", 0.02)
        rho = kw.get("rho", 0.9)
        w = rw.standard_normal((n_out, n_in)) * w_std
        n_outl = kw.get("outlier_cols", 0)
        if n_outl:
            cols = rw.choice(n_in, size=n_outl, replace=False)
            w[:, cols] *= kw.get("outlier_scale", 20.0)
        scale_sigma = kw.get("scale_sigma", 0.0)
        s = np.exp(rs.standard_normal(n_in) * scale_sigma) if scale_sigma > 0 else None
        xs = []
        for r, m in zip(chunk_rngs, chunk_sizes):
            x = _ar1_rows(r, m, n_in, rho)
            if s is not None:
                x *= s[None, :]
            xs.append(x)
        return _finish(name, dtype, w, xs, targets)

    if recipe in ("spiked", "lmhead"):
        rank = kw.get("rank", 64)
        if recipe == "spiked":
            nu = kw.get("nu", 5.0)
            w = _student_t(rw, nu, (n_out, n_in), kw.get("w_std", 0.02))
        else:
            s_zipf = kw.get("zipf_s", 1.1)
            p = (np.arange(1, n_out + 1, dtype=np.float64)) ** (-s_zipf)
            p /= p.sum()
            sig = p ** (-0.25)
            sig *= kw.get("w_rms", 0.02) / math.sqrt(np.mean(sig * sig))
            w = rw.standard_normal((n_out, n_in)) * sig[:, None]
        v, lam, d = _spiked_factors(rs, n_in, rank)
        xs = []
        for r, m in zip(chunk_rngs, chunk_sizes):
            za = r.standard_normal((m, rank))
            zb = r.standard_normal((m, n_in))
            xs.append((za * np.sqrt(lam)[None, :]) @ v.T + zb * np.sqrt(d)[None, :])
        return _finish(name, dtype, w, xs, targets)

    if recipe == "blockar1":
        nu = kw.get("nu", 4.0)
        block = kw.get("block", 512)
        rho = kw.get("rho", 0.9)
        w = _student_t(rw, nu, (n_out, n_in), kw.get("w_std", 0.01))
        dscale = np.exp(rs.standard_normal(n_in))
        xs = [_ar1_rows(r, m, n_in, rho, block) * dscale[None, :] for r, m in zip(chunk_rngs, chunk_sizes)]
        return _finish(name, dtype, w, xs, targets)

    raise ValueError(f"unknown recipe {recipe!r}")


# The five named workloads: the pages' layer shapes (attention projection, MLP up/down
# projection, LM head) with synthetic weights and activations of the stated structure.
NAMED = {
    "ar1_256": dict(recipe="ar1", n_out=256, n_in=256, n_rows=1024, dtype="f32", targets=(2.0,),
                    w_std=0.02, rho=0.9),
    "attn_4096": dict(recipe="spiked", n_out=4096, n_in=4096, n_rows=8192, dtype="bf16",
                      targets=(1.0, 2.0, 3.0, 4.0), nu=5.0, w_std=0.02, rank=64),
    "mlp_up_11008x4096": dict(recipe="ar1", n_out=11008, n_in=4096, n_rows=16384, dtype="bf16",
                              targets=(2.0,), w_std=0.015, rho=0.95, scale_sigma=0.5,
                              outlier_cols=4, outlier_scale=20.0),
    "lmhead_32000x4096": dict(recipe="lmhead", n_out=32000, n_in=4096, n_rows=8192, dtype="bf16",
                              targets=(1.5, 3.0), zipf_s=1.1, w_rms=0.02, rank=256),
    "mlp_down_8192x28672": dict(recipe="blockar1", n_out=8192, n_in=28672, n_rows=32768, dtype="bf16",
                                targets=(2.0,), chunk_rows=4096, nu=4.0, w_std=0.01, block=512, rho=0.9),
}


def named_workload(name: str, seed: int = 0, **override) -> Layer:
    spec = dict(NAMED[name])
    spec.update(override)
    recipe = spec.pop("recipe")
    n_out, n_in, n_rows = spec.pop("n_out"), spec.pop("n_in"), spec.pop("n_rows")
    return make_layer(recipe, n_out, n_in, n_rows, seed=seed, name=name, **spec)


def iter_x_chunks(layer: Layer) -> Iterator[np.ndarray]:
    yield from layer.x_chunks
