"""GPU parity of the entropy coder through the C ABI: the device container equals the reference
container (oracle/rans.py) byte for byte, decoding returns the codes, decoding to weights equals
the dequantization of wsic_distortion bit for bit, the coded size of real SIC codes sits just
above their empirical entropy, and a damaged container is rejected without faulting."""
import numpy as np
import pytest
import torch

import oracle
from oracle import rans
from parity import DEV, say, w_tensor
from rate_allocated_weight_amd import _lib as lib
from rate_allocated_weight_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lib.lib()
    return torch.device(DEV)


def _codes(seed, n, spread, esc=0):
    rng = np.random.default_rng(seed)
    q = np.rint(rng.standard_normal(n) * spread).astype(np.int64)
    if esc:
        pos = rng.choice(n, esc, replace=False)
        q[pos] = rng.choice([5000, -70000, 2 ** 31 - 1, -(2 ** 31) + 1, 2048, -2048], esc)
    return q.astype(np.int32)


@pytest.mark.parametrize("n,spread,esc,L", [(5000, 2.0, 0, 16), (7777, 30.0, 9, 8), (640, 0.3, 0, 4),
                                            (64 * 8 * 3, 700.0, 3, 8), (1, 1.0, 0, 4), (20000, 0.0, 0, 32)])
def test_container_matches_reference(device, n, spread, esc, L):
    q = _codes(n, n, spread, esc)
    qt = torch.from_numpy(q).to(DEV)
    blob, nb = lib.rans_encode(qt, L)
    ref = rans.encode(q, L)
    dev = blob[:nb].cpu().numpy().tobytes()
    assert nb == len(ref)
    assert dev == ref
    back = lib.rans_decode(blob, nb, n)
    np.testing.assert_array_equal(back.cpu().numpy(), q)


@pytest.mark.parametrize("R", [1.0, 2.0, 4.0])
def test_sic_codes_coded_size(device, R):
    layer = workloads.make_layer("spiked", 300, 333, 900, seed=0, name="spiked_300x333", dtype="bf16", rank=16)
    L, info = oracle.cholesky_lower(oracle.covariance(layer.x_chunks))
    U = torch.from_numpy(np.ascontiguousarray(L.T)).to(DEV)
    Wt = w_tensor(layer)
    wf = lib.waterfill(Wt, U, R)
    codes = wf["codes"].contiguous()
    blob, nb = lib.rans_encode(codes, 64)
    back = lib.rans_decode(blob, nb, codes.numel()).view_as(codes)
    assert torch.equal(back, codes)
    n = codes.numel()
    bits = 8.0 * nb / n
    say(f"[rans] R={R}: entropy {wf['rate']:.4f}, container {bits:.4f} bits per code ({nb} bytes)")
    assert bits >= wf["rate"]
    # the excess: the 2^14 table's cross-entropy loss, 32 bits of state per stream, the headers
    streams = 64 * ((n + 64 * 64 - 1) // (64 * 64))
    assert bits <= wf["rate"] * 1.01 + (32.0 * streams + 8192.0) / n
    # decoding straight to weights equals the dequantization of the distortion call, bit for bit
    for dt in (torch.float32, torch.bfloat16):
        _, w_ref = lib.distortion(Wt, codes, U, wf["c"], resid=wf["resid"], w_hat_dtype=dt)
        w = lib.rans_decode_dequant(blob, nb, layer.n_out, layer.n_in, U, wf["c"], dtype=dt)
        assert torch.equal(w.view(torch.int16) if dt == torch.bfloat16 else w.view(torch.int32),
                           w_ref.view(torch.int16) if dt == torch.bfloat16 else w_ref.view(torch.int32))


def test_damaged_container_is_rejected(device):
    q = _codes(9, 30000, 5.0, 4)
    qt = torch.from_numpy(q).to(DEV)
    blob, nb = lib.rans_encode(qt, 32)
    with pytest.raises(lib.WsicError):  # wrong length
        lib.rans_decode(blob, nb, q.size - 1)
    bad = blob.clone()
    bad[0] ^= 0xFF  # magic
    with pytest.raises(lib.WsicError):
        lib.rans_decode(bad, nb, q.size)
    with pytest.raises(lib.WsicError):  # truncated
        lib.rans_decode(blob, nb - 100, q.size)
    bad = blob.clone()
    bad[nb - 2000:nb - 1000] ^= 0x5A  # payload bytes: streams no longer end in their start state
    with pytest.raises(lib.WsicError):
        lib.rans_decode(bad, nb, q.size)
