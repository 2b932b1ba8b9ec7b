"""Shared helpers of the GPU parity tests: move seeded workloads to the device and grade
code agreement against the oracle."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

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


def host_workers(n_in: int) -> int:
    """Oracle worker threads: the host cores this process may use (at most 16), fewer for very
    wide layers, where every oracle call holds an n_in x n_in fp64 interference matrix."""
    cores = len(os.sched_getaffinity(0))
    w = min(16, cores)
    if n_in > 8192:
        w = min(w, 4)
    return max(1, w)


def grade_rows(w: np.ndarray, L: np.ndarray, c: float, q_dev: np.ndarray, r_dev=None, sigma=None,
               rows=None, chunk: int = 0, workers: int = 0):
    """Grade the device's codes on every row (or on `rows`) against the oracle's SIC at the same
    factor and grid scale. Rows are independent, so the oracle runs on row chunks in a thread
    pool, each thread with one BLAS thread (the oracle's column loop is a matrix-vector product
    per column, which scales better across chunks than inside one BLAS call).

    w: the layer's weights (host, all rows); L: lower factor (U^T of the device's U);
    q_dev / r_dev: the device's codes / residuals for the graded rows (host arrays, same row
    order as `rows`); sigma: host covariance for each row's direct distortion e Sigma e^T.

    Returns a dict: n, exact, tie, bad, bad_rows (first few), max_dr (max |r_dev - r_or| /
    alpha over exact rows), d_rows (the oracle's e Sigma e^T per graded row, if sigma)."""
    import oracle
    from threadpoolctl import threadpool_limits

    rows = np.arange(w.shape[0]) if rows is None else np.asarray(rows)
    n = len(rows)
    n_in = w.shape[1]
    workers = workers or host_workers(n_in)
    if not chunk:
        chunk = int(min(1024, max(32, -(-n // (4 * workers)))))
    starts = list(range(0, n, chunk))

    def one(s):
        idx = rows[s:s + chunk]
        sic = oracle.sic_quantize(w[idx], L, c)
        qd = np.asarray(q_dev[s:s + chunk], dtype=np.int64)
        ex, ti, bd = grade_codes(qd, sic)
        diff = np.any(qd != sic["q"], axis=1)
        bad_list = [int(idx[i]) for i in np.where(diff)[0]][:8]
        mdr = 0.0
        if r_dev is not None and (~diff).any():
            rd = np.asarray(r_dev[s:s + chunk], dtype=np.float64)[~diff]
            mdr = float((np.abs(rd - sic["r"][~diff]) / sic["alpha"][None, :]).max())
        dr = None
        if sigma is not None:
            e = sic["e"]
            dr = np.einsum("ij,ij->i", e @ sigma, e)
        return ex, ti, bd, bad_list, mdr, dr

    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            parts = list(ex.map(one, starts))
    out = dict(n=n, exact=sum(p[0] for p in parts), tie=sum(p[1] for p in parts),
               bad=sum(p[2] for p in parts), bad_rows=[r for p in parts for r in p[3]][:8],
               max_dr=max(p[4] for p in parts), workers=workers, chunk=chunk)
    if sigma is not None:
        out["d_rows"] = np.concatenate([p[5] for p in parts])
    return out


def assert_rows_graded(g: dict, label: str = ""):
    """The parity bar on a full grading: no mismatch that is not a tie-flip, at least 99.9 %
    of rows bit-exact."""
    say(f"  codes {label}: rows exact {g['exact']}/{g['n']}, tie-flips {g['tie']}, mismatches "
        f"{g['bad']} (oracle on {g['workers']} threads, {g['chunk']} rows per chunk)"
        + (f"; differing rows {g['bad_rows']}" if g['bad'] or g['tie'] else ""))
    assert g["bad"] == 0
    assert g["exact"] >= ROW_EXACT_MIN * g["n"]
