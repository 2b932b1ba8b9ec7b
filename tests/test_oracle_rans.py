"""Pins of the reference entropy coder (oracle/rans.py): lossless round trips, the table, the
Shannon bound and the exact cost of a uniform source."""
import numpy as np
import pytest

import oracle
from oracle import rans


def _codes(seed, n, spread, esc=0):
    rng = np.random.default_rng(seed)
    q = np.rint(rng.standard_normal(n) * spread).astype(np.int64)
    if esc:
        pos = rng.choice(n, esc, replace=False)
        q[pos] = rng.choice([5000, -70000, 2 ** 31 - 1, -(2 ** 31) + 1, 2048, -2048], esc)
    return q


@pytest.mark.parametrize("n,spread,esc,L", [(5000, 2.0, 0, 16), (7777, 30.0, 9, 8), (640, 0.3, 0, 4),
                                            (64 * 8 * 3, 700.0, 3, 8), (1, 1.0, 0, 4)])
def test_roundtrip(n, spread, esc, L):
    q = _codes(n, n, spread, esc)
    blob = rans.encode(q, L)
    np.testing.assert_array_equal(rans.decode(blob), q)


def test_table_invariants():
    q = _codes(1, 20000, 12.0, 5)
    lo, f = rans.build_table(q)
    assert f.sum() == rans.M
    inw = q[(q >= -rans.WINDOW) & (q <= rans.WINDOW)]
    present = np.unique(inw) - lo
    assert np.all(f[present] >= 1)
    absent = np.setdiff1d(np.arange(f.size - 1), present)
    assert np.all(f[absent] == 0)
    assert f[-1] >= 1  # escapes present


def _total_bits(blob):
    h = np.frombuffer(blob[:64], dtype=np.uint32)
    groups, words = int(h[5]), int(h[10])
    return 16 * words + 32 * 64 * groups


def test_shannon_bound_and_overhead():
    """A static-table code cannot beat the empirical entropy; with a 2^14 table its excess over
    it is the table's cross-entropy loss plus 32 bits of final state per lane."""
    q = _codes(2, 64 * 256 * 4, 3.0)
    blob = rans.encode(q, 256)
    H = oracle.entropy_bits(q)
    bits = _total_bits(blob)
    assert bits >= q.size * H
    assert bits <= q.size * H * 1.01 + 32 * 64 * 4


def test_uniform_source_costs_k_bits():
    """2^k equally frequent symbols get frequency M / 2^k each and cost exactly k bits: the
    payload holds k N bits less what the final states carry above their floor 2^16 (at most 16
    bits per stream)."""
    k = 5
    q = np.tile(np.arange(2 ** k) - 9, 64 * 64)
    np.random.default_rng(3).shuffle(q)
    lo, f = rans.build_table(q)
    assert np.all(f[:-1] == rans.M >> k)
    blob = rans.encode(q, 64)
    h = np.frombuffer(blob[:64], dtype=np.uint32)
    streams = 64 * int(h[5])
    payload_bits = 16 * int(h[10])
    assert k * q.size - 16 * streams <= payload_bits <= k * q.size
