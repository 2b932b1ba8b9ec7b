"""Shared helpers of the GPU parity tests: move seeded workloads to the device and grade
code agreement against the oracle."""
import sys

import numpy as np
import torch

from rate_allocated_weight_amd import _lib as lib

DEV = "cuda:0"

# tolerances of the parity bar
ROW_EXACT_MIN = 0.999   # fraction of rows whose codes must be bit-exact
TIE_DIST = 1e-5         # a differing row must first differ where the oracle is this close to a tie
RATE_TOL = 1e-4         # bits per weight
REL_TOL = 1e-3          # grid scale and distortion


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def w_tensor(layer, device=DEV):
    if layer.dtype == "bf16":
        return lib.bf16_from_bits(layer.w_bits, device)
    return torch.from_numpy(layer.w).to(device)


def x_tensors(layer, device=DEV):
    if layer.dtype == "bf16":
        return [lib.bf16_from_bits(b, device) for b in layer.x_bits_chunks]
    return [torch.from_numpy(c).to(device) for c in layer.x_chunks]


def grade_codes(q_gpu: np.ndarray, sic: dict, rows=None):
    """Compare device codes with oracle SIC output (dict from oracle.sic_quantize).

    Returns (n_exact, n_tie, n_bad). A row that differs counts as a tie-flip when, at its first
    differing column in processing order (the largest index), the oracle's scaled target
    t/alpha lies within TIE_DIST of a rounding boundary."""
    q_or = sic["q"]
    q_gpu = np.asarray(q_gpu, dtype=np.int64)
    if rows is not None:
        q_gpu = q_gpu[rows]
    assert q_gpu.shape == q_or.shape
    diff = q_gpu != q_or
    bad_rows = np.where(diff.any(axis=1))[0]
    n_tie = 0
    n_bad = 0
    z = sic["t"] / sic["alpha"][None, :]
    for r in bad_rows:
        j = np.where(diff[r])[0].max()
        frac = z[r, j] - np.floor(z[r, j])
        if abs(frac - 0.5) < TIE_DIST:
            n_tie += 1
        else:
            n_bad += 1
    return q_or.shape[0] - len(bad_rows), n_tie, n_bad


def assert_codes_parity(q_gpu, sic, rows=None, label=""):
    n_exact, n_tie, n_bad = grade_codes(q_gpu, sic, rows)
    n = n_exact + n_tie + n_bad
    say(f"  codes {label}: rows exact {n_exact}/{n}, tie-flips {n_tie}, mismatches {n_bad}")
    assert n_bad == 0
    assert n_exact >= ROW_EXACT_MIN * n
    return n_exact, n_tie, n_bad
