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


@pytest.mark.parametrize("n,spread,esc,L", [(64 * 1024 * 2 + 4321, 30.0, 17, 1024),
                                            (64 * 300 * 5 + 11, 3.0, 0, 300),
                                            (64 * 1000 + 5, 400.0, 5, 1000),
                                            (64 * 2048, 1.0e4, 0, 2048),
                                            (64 * 8 * 1100 + 3, 2.0, 5, 8),
                                            (200, 2.0, 1, 1),
                                            (64 * 65536, 2.0, 3, 65536)])
def test_long_streams_match_reference(device, n, spread, esc, L):
    """Streams long enough that the decoder refills its payload ring many times, stream lengths that
    are not a multiple of the kernels' step blocks, a rate near 10 bits, a source that is mostly
    escapes, 1101 short groups (138 decoder workgroups), and both ends of the stream length (one
    code per stream; 65536, the largest, in a single group of 4.2 M codes): containers equal the
    reference's byte for byte and decode back to the codes."""
    q = _codes(n + 1, n, spread, esc)
    qt = torch.from_numpy(q).to(DEV)
    blob, nb = lib.rans_encode(qt, L)
    ref = rans.encode(q, L)
    say(f"[rans-long] n={n} L={L} spread={spread}: {8.0 * len(ref) / n:.3f} bits per code")
    assert nb == len(ref)
    assert blob[:nb].cpu().numpy().tobytes() == ref
    back = lib.rans_decode(blob, nb, n)
    np.testing.assert_array_equal(back.cpu().numpy(), q)


@pytest.mark.parametrize("L", [37, 1000])
def test_decode_to_weights_long_streams(device, L):
    """Decoding to weights with streams whose length is not a multiple of the step blocks (the
    column scales are loaded a block ahead) and with many ring refills (4 bits per code, 1000
    codes per stream) equals the dequantization of wsic_distortion bit for bit."""
    layer = workloads.make_layer("spiked", 300, 333, 900, seed=0, name="spiked_300x333", dtype="bf16", rank=16)
    Lc, info = oracle.cholesky_lower(oracle.covariance(layer.x_chunks))
    U = torch.from_numpy(np.ascontiguousarray(Lc.T)).to(DEV)
    Wt = w_tensor(layer)
    wf = lib.waterfill(Wt, U, 4.0)
    codes = wf["codes"].contiguous()
    blob, nb = lib.rans_encode(codes, L)
    assert blob[:nb].cpu().numpy().tobytes() == rans.encode(codes.cpu().numpy().ravel(), L)
    for dt in (torch.float32, torch.bfloat16):
        _, w_ref = lib.distortion(Wt, codes, U, wf["c"], resid=wf["resid"], w_hat_dtype=dt)
        w = lib.rans_decode_dequant(blob, nb, layer.n_out, layer.n_in, U, wf["c"], dtype=dt)
        assert torch.equal(w.view(torch.int16) if dt == torch.bfloat16 else w.view(torch.int32),
                           w_ref.view(torch.int16) if dt == torch.bfloat16 else w_ref.view(torch.int32))


def test_decode_to_weights_wide_rows(device):
    """More than 4096 columns: the column scales no longer fit beside the decoder's tables in LDS
    and are loaded a block of steps ahead instead; the weights still equal the dequantization of
    wsic_distortion bit for bit, for whole and ragged stream blocks."""
    n_out, n_in = 24, 4500
    rng = np.random.default_rng(7)
    codes = torch.from_numpy(_codes(11, n_out * n_in, 3.0).reshape(n_out, n_in)).to(DEV)
    U = torch.diag(torch.from_numpy(rng.uniform(0.5, 2.0, n_in))).to(DEV)
    W = torch.zeros(n_out, n_in, dtype=torch.float32, device=DEV)
    c = 0.0123
    for L in (1000, 37):
        blob, nb = lib.rans_encode(codes, L)
        for dt in (torch.float32, torch.bfloat16):
            _, w_ref = lib.distortion(W, codes, U, c, mode="direct", w_hat_dtype=dt)
            w = lib.rans_decode_dequant(blob, nb, n_out, n_in, U, c, dtype=dt)
            assert torch.equal(w.view(torch.int16) if dt == torch.bfloat16 else w.view(torch.int32),
                               w_ref.view(torch.int16) if dt == torch.bfloat16 else w_ref.view(torch.int32))


def test_decode_to_weights_rejects_bad_diagonal(device):
    """A zero or NaN diagonal entry of U is reported (its check travels with the decode's own
    verdict), and a good U decodes correctly right after."""
    n_out, n_in = 40, 70
    q = _codes(5, n_out * n_in, 2.0).reshape(n_out, n_in)
    codes = torch.from_numpy(q).to(DEV)
    blob, nb = lib.rans_encode(codes, 16)
    for bad in (0.0, float("nan")):
        U = torch.eye(n_in, dtype=torch.float64, device=DEV)
        U[3, 3] = bad
        with pytest.raises(lib.WsicError):
            lib.rans_decode_dequant(blob, nb, n_out, n_in, U, 0.01, dtype=torch.float32)
    d = np.linspace(0.5, 2.0, n_in)
    U = torch.diag(torch.from_numpy(d)).to(DEV)
    w = lib.rans_decode_dequant(blob, nb, n_out, n_in, U, 0.01, dtype=torch.float32)
    ref = ((0.01 * (1.0 / d))[None, :] * q.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(w.cpu().numpy(), ref)


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
    bad = blob.clone()
    bad[64] ^= 0x01  # the first frequency: the table no longer sums to 2^14
    with pytest.raises(lib.WsicError):
        lib.rans_decode(bad, nb, q.size)
    bad = blob.clone()
    bad[64:64 + 40] = 0xFF  # frequencies far above 2^14
    with pytest.raises(lib.WsicError):
        lib.rans_decode(bad, nb, q.size)
    # sections located from the header (groups G, symbols nsym): word offsets pointing far past
    # the payload, and scrambled initial states; every read stays bounded and the decode fails
    hdr = np.frombuffer(blob[:64].cpu().numpy().tobytes(), dtype="<u4")
    G, nsym = int(hdr[5]), int(hdr[7])
    a16 = lambda v: (v + 15) // 16 * 16
    gofs = a16(64 + 2 * nsym)
    states = a16(a16(gofs + 4 * (G + 1)) + 4 * (G + 1))
    bad = blob.clone()
    bad[gofs + 4:gofs + 4 * G] = 0xF0
    with pytest.raises(lib.WsicError):
        lib.rans_decode(bad, nb, q.size)
    bad = blob.clone()
    bad[states:states + 4 * 64 * G] ^= 0x3C
    with pytest.raises(lib.WsicError):
        lib.rans_decode(bad, nb, q.size)
