"""ctypes binding of libwsic (the C ABI in include/wsic.h).

Argument marshalling only: every step runs in the HIP library. Tensors must live on a ROCm
device; workspaces are allocated here with torch and handed to the library. There is no CPU
fallback: importing succeeds without a GPU, but any call raises if libwsic.so is missing.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwsic.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "wsic.h")

OK, E_INVAL, E_NOT_PD, E_NONFINITE, E_NO_BRACKET, E_RANGE, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16 = 0, 1
(OP_COVARIANCE, OP_CHOLESKY, OP_SIC, OP_WATERFILL, OP_ENTROPY, OP_DISTORTION, OP_CURVATURE,
 OP_SOFTWATER, OP_SOFTWATER_DIST, OP_ENTROPY_COLUMNS, OP_GAUSS_RATE, OP_LMMSE, OP_LIVE, OP_RANS_ENC,
 OP_RANS_DEC) = range(15)
RATE_POOLED, RATE_COLUMNS = 0, 1
_RATE_MODES = {"pooled": RATE_POOLED, "columns": RATE_COLUMNS}
D_RESID, D_DIRECT = 0, 1
WF_AUTO, WF_SECANT, WF_BISECT = 0, 1, 2
# diagnostic switches (wsic_debug_set)
DEBUG_KNOBS = {"fp64_product": 0, "super_blocks": 1, "guard_scale": 2, "chol_fused": 3,
               "logits_generic": 4, "trace": 5, "probe": 6}

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_d = ctypes.c_double
_sz = ctypes.c_size_t


class WsicError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status_name(status)}]")
        self.status = status
        self.message = message


class WfOpts(ctypes.Structure):
    _fields_ = [("rate_tol", ctypes.c_double), ("bracket_log2", ctypes.c_double),
                ("max_passes", ctypes.c_int32), ("mode", ctypes.c_int32), ("c_init", ctypes.c_double),
                ("rate_mode", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_SIGS = {
    "wsic_version": (ctypes.c_int, []),
    "wsic_last_error": (ctypes.c_char_p, []),
    "wsic_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "wsic_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64]),
    "wsic_covariance": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _d, _d, _p, _i64, _p, _sz, _p]),
    "wsic_cholesky": (ctypes.c_int, [_p, _i64, _i64, ctypes.POINTER(_i64), _p, _sz, _p]),
    "wsic_sic_quantize": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _d, _p, _i64, _p,
                                         _i64, _p, _sz, _p]),
    "wsic_waterfill": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _d, ctypes.POINTER(WfOpts),
                                      ctypes.POINTER(_d), ctypes.POINTER(_d), ctypes.POINTER(ctypes.c_int32),
                                      _p, _i64, _p, _i64, _p, _sz, _p]),
    "wsic_entropy": (ctypes.c_int, [_p, _i64, _i64, _i64, ctypes.POINTER(_d), ctypes.POINTER(_i64), _p, _sz, _p]),
    "wsic_distortion": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _d, _p, _i64,
                                       ctypes.c_int, ctypes.POINTER(_d), _p, ctypes.c_int, _i64, _p, _sz, _p]),
    "wsic_softmax_curvature": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _d, _d, _d,
                                              _p, _p, _sz, _p]),
    "wsic_softwater_waterfill": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _d,
                                                ctypes.POINTER(WfOpts), ctypes.POINTER(_d), ctypes.POINTER(_d),
                                                ctypes.POINTER(ctypes.c_int32), _p, _i64, _p, _i64, _p, _sz, _p]),
    "wsic_softwater_distortion": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i64, _d, _p, _p, _i64,
                                                 ctypes.POINTER(_d), _p, ctypes.c_int, _i64, _p, _sz, _p]),
    "wsic_entropy_columns": (ctypes.c_int, [_p, _i64, _i64, _i64, ctypes.POINTER(_d), _p, _sz, _p]),
    "wsic_gaussian_rate": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _d, ctypes.POINTER(_d),
                                          ctypes.POINTER(_d), _p, _sz, _p]),
    "wsic_lmmse_scale": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _p,
                                        ctypes.POINTER(_d), ctypes.POINTER(_d), _p, _sz, _p]),
    "wsic_live_features": (ctypes.c_int, [_p, _i64, _i64, _d, _p, _p, ctypes.POINTER(_i64), _p, _sz, _p]),
    "wsic_gather_features": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64,
                                            _p, _i64, _p]),
    "wsic_scatter_codes": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "wsic_rans_bound": (_sz, [_i64, ctypes.c_int32]),
    "wsic_rans_encode": (ctypes.c_int, [_p, _i64, ctypes.c_int32, _p, _sz, ctypes.POINTER(_sz), _p, _sz, _p]),
    "wsic_rans_decode": (ctypes.c_int, [_p, _sz, _p, _i64, _p, _sz, _p]),
    "wsic_rans_decode_dequant": (ctypes.c_int, [_p, _sz, _i64, _i64, _p, _i64, _d, _p, ctypes.c_int, _p, _sz, _p]),
    "wsic_distortion_noalloc": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _d, _p,
                                               _i64, ctypes.c_int, ctypes.POINTER(_d), _p, ctypes.c_int, _i64, _p]),
    "wsic_debug_set": (ctypes.c_int, [ctypes.c_int, _d]),
    "wsic_debug_get": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(_d)]),
    "wsic_debug_reset": (None, []),
    "wsic_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "wsic_profile_reset": (ctypes.c_int, []),
    "wsic_profile_select": (ctypes.c_int, [ctypes.c_char_p]),
    "wsic_profile_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(_i64), ctypes.POINTER(_d),
                                         ctypes.POINTER(_d)]),
    "wsic_profile_names": (ctypes.c_int, [ctypes.c_char_p, _sz]),
}

_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libwsic.so (built in-tree by rate_allocated_weight_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m rate_allocated_weight_amd.build` (there is no CPU fallback)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = h
    return _LIB


def header_functions() -> List[str]:
    """Names of the functions declared in include/wsic.h."""
    txt = open(HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wsic_[a-z_0-9]+)\s*\(", txt)))


def status_name(s: int) -> str:
    try:
        return lib().wsic_status_str(s).decode()
    except ImportError:
        return str(s)


def _check(status: int) -> None:
    if status != OK:
        msg = lib().wsic_last_error().decode()
        raise WsicError(status, msg)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libwsic works on device tensors only")


def _rowmajor(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def workspace_bytes(op: int, n_out: int, n_in: int) -> int:
    return int(lib().wsic_workspace_bytes(op, n_out, n_in))


def workspace(op: int, n_out: int, n_in: int, device) -> torch.Tensor:
    nb = workspace_bytes(op, n_out, n_in)
    if nb == 0:
        raise ValueError("bad workspace query")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _ws_args(ws: torch.Tensor):
    return ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel())


# ------------------------------------------------------------------------------ entry points
def covariance(X: torch.Tensor, sigma: Optional[torch.Tensor] = None, alpha: float = 1.0,
               beta: float = 0.0, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sigma <- beta*Sigma + alpha*X^T X (fp64, full symmetric)."""
    _need_cuda(X)
    ldx = _rowmajor(X)
    rows, n = X.shape
    if sigma is None:
        sigma = torch.empty((n, n), dtype=torch.float64, device=X.device)
    ws = ws if ws is not None else workspace(OP_COVARIANCE, 1, n, X.device)
    _check(lib().wsic_covariance(_p(X.data_ptr()), _dtype_code(X), rows, n, ldx, alpha, beta,
                                 _p(sigma.data_ptr()), _rowmajor(sigma), *_ws_args(ws), _stream(X)))
    return sigma


def covariance_chunks(chunks: Sequence[torch.Tensor]) -> torch.Tensor:
    """Sigma = X^T X / N over streamed row chunks."""
    n_total = sum(int(c.shape[0]) for c in chunks)
    sigma = None
    ws = None
    for i, c in enumerate(chunks):
        if ws is None:
            ws = workspace(OP_COVARIANCE, 1, c.shape[1], c.device)
        sigma = covariance(c, sigma, alpha=1.0 / n_total, beta=0.0 if i == 0 else 1.0, ws=ws)
    return sigma


def cholesky(A: torch.Tensor, ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """In place: upper(A) <- U with Sigma = U^T U, lower zeroed. Returns (A, info); raises on
    failure with the pivot in the message."""
    _need_cuda(A)
    if A.dtype != torch.float64:
        raise TypeError("cholesky expects float64")
    n = A.shape[0]
    ws = ws if ws is not None else workspace(OP_CHOLESKY, 1, n, A.device)
    info = _i64(0)
    st = lib().wsic_cholesky(_p(A.data_ptr()), n, _rowmajor(A), ctypes.byref(info), *_ws_args(ws), _stream(A))
    if st == E_NOT_PD:
        err = WsicError(st, lib().wsic_last_error().decode())
        err.info = int(info.value)
        raise err
    _check(st)
    return A, int(info.value)


def sic_quantize(W: torch.Tensor, U: torch.Tensor, c: float, want_resid: bool = False,
                 codes: Optional[torch.Tensor] = None, resid: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None):
    """One SIC pass at grid scale c. Returns (codes int32, resid float32 or None)."""
    _need_cuda(W, U)
    n_out, n_in = W.shape
    if codes is None:
        codes = torch.empty((n_out, n_in), dtype=torch.int32, device=W.device)
    if want_resid and resid is None:
        resid = torch.empty((n_out, n_in), dtype=torch.float32, device=W.device)
    ws = ws if ws is not None else workspace(OP_SIC, n_out, n_in, W.device)
    _check(lib().wsic_sic_quantize(
        _p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(U.data_ptr()), _rowmajor(U), float(c),
        _p(codes.data_ptr()), _rowmajor(codes), _p(resid.data_ptr() if resid is not None else 0),
        _rowmajor(resid) if resid is not None else n_in, *_ws_args(ws), _stream(W)))
    return codes, resid


_MODES = {"auto": WF_AUTO, "secant": WF_SECANT, "bisect": WF_BISECT}


def waterfill(W: torch.Tensor, U: torch.Tensor, target_bits: float, *, mode: str = "auto",
              rate_tol: float = 8e-5, bracket_log2: float = 2.0 ** -20, max_passes: int = 64,
              c_init: float = 0.0, want_resid: bool = True, codes: Optional[torch.Tensor] = None,
              resid: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
              rate_mode: str = "pooled") -> Dict[str, object]:
    """Grid scale c with code entropy H(c) <= target_bits (pooled, or the mean column entropy),
    and its codes."""
    _need_cuda(W, U)
    n_out, n_in = W.shape
    if codes is None:
        codes = torch.empty((n_out, n_in), dtype=torch.int32, device=W.device)
    if want_resid and resid is None:
        resid = torch.empty((n_out, n_in), dtype=torch.float32, device=W.device)
    ws = ws if ws is not None else workspace(OP_WATERFILL, n_out, n_in, W.device)
    opts = WfOpts(rate_tol, bracket_log2, max_passes, _MODES[mode], c_init, _RATE_MODES[rate_mode], 0)
    c_out, rate_out, passes = _d(0), _d(0), ctypes.c_int32(0)
    _check(lib().wsic_waterfill(
        _p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(U.data_ptr()), _rowmajor(U),
        float(target_bits), ctypes.byref(opts), ctypes.byref(c_out), ctypes.byref(rate_out), ctypes.byref(passes),
        _p(codes.data_ptr()), _rowmajor(codes), _p(resid.data_ptr() if resid is not None else 0),
        _rowmajor(resid) if resid is not None else n_in, *_ws_args(ws), _stream(W)))
    return {"c": c_out.value, "rate": rate_out.value, "passes": int(passes.value), "codes": codes,
            "resid": resid}


def entropy(codes: torch.Tensor, ws: Optional[torch.Tensor] = None) -> Tuple[float, int]:
    """Pooled empirical entropy (bits per code) and number of distinct codes."""
    _need_cuda(codes)
    if codes.dtype != torch.int32:
        raise TypeError("codes must be int32")
    n_out, n_in = codes.shape
    ws = ws if ws is not None else workspace(OP_ENTROPY, n_out, n_in, codes.device)
    h, ns = _d(0), _i64(0)
    _check(lib().wsic_entropy(_p(codes.data_ptr()), n_out, n_in, _rowmajor(codes), ctypes.byref(h),
                              ctypes.byref(ns), *_ws_args(ws), _stream(codes)))
    return h.value, int(ns.value)


def entropy_columns(codes: torch.Tensor, ws: Optional[torch.Tensor] = None) -> float:
    """Mean over columns of each column's code entropy (bits per code)."""
    _need_cuda(codes)
    if codes.dtype != torch.int32:
        raise TypeError("codes must be int32")
    n_out, n_in = codes.shape
    ws = ws if ws is not None else workspace(OP_ENTROPY_COLUMNS, n_out, n_in, codes.device)
    h = _d(0)
    _check(lib().wsic_entropy_columns(_p(codes.data_ptr()), n_out, n_in, _rowmajor(codes), ctypes.byref(h),
                                      *_ws_args(ws), _stream(codes)))
    return h.value


def gaussian_rate(W: torch.Tensor, U: torch.Tensor, D: float, ws: Optional[torch.Tensor] = None):
    """High-rate Gaussian limit (bits per weight) at total distortion D, and the weight variance."""
    _need_cuda(W, U)
    n_out, n_in = W.shape
    ws = ws if ws is not None else workspace(OP_GAUSS_RATE, n_out, n_in, W.device)
    r, v = _d(0), _d(0)
    _check(lib().wsic_gaussian_rate(_p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(U.data_ptr()),
                                    _rowmajor(U), float(D), ctypes.byref(r), ctypes.byref(v), *_ws_args(ws),
                                    _stream(W)))
    return r.value, v.value


def lmmse_scale(W: torch.Tensor, U: torch.Tensor, resid: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """Per-row LMMSE factors gamma (device, float64) and the distortion before and after."""
    _need_cuda(W, U, resid)
    n_out, n_in = W.shape
    gamma = torch.empty(n_out, dtype=torch.float64, device=W.device)
    ws = ws if ws is not None else workspace(OP_LMMSE, n_out, n_in, W.device)
    db, da = _d(0), _d(0)
    _check(lib().wsic_lmmse_scale(_p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(U.data_ptr()),
                                  _rowmajor(U), _p(resid.data_ptr()), _rowmajor(resid), _p(gamma.data_ptr()),
                                  ctypes.byref(db), ctypes.byref(da), *_ws_args(ws), _stream(W)))
    return gamma, db.value, da.value


def live_features(sigma: torch.Tensor, tau: float):
    """(idx, pos, n_live): live input columns (Sigma_ii > tau max Sigma_jj) and the inverse map."""
    _need_cuda(sigma)
    n = sigma.shape[0]
    idx = torch.empty(n, dtype=torch.int32, device=sigma.device)
    pos = torch.empty(n, dtype=torch.int32, device=sigma.device)
    ws = workspace(OP_LIVE, 0, n, sigma.device)
    nl = _i64(0)
    _check(lib().wsic_live_features(_p(sigma.data_ptr()), n, _rowmajor(sigma), float(tau), _p(idx.data_ptr()),
                                    _p(pos.data_ptr()), ctypes.byref(nl), *_ws_args(ws), _stream(sigma)))
    return idx, pos, int(nl.value)


def gather_features(W: torch.Tensor, idx: torch.Tensor, n_live: int, sigma: Optional[torch.Tensor] = None):
    """W[:, idx[:n_live]] and, if given, sigma[idx][:, idx]."""
    _need_cuda(W, idx)
    n_out, n_in = W.shape
    Wl = torch.empty((n_out, n_live), dtype=W.dtype, device=W.device)
    Sl = torch.empty((n_live, n_live), dtype=torch.float64, device=W.device) if sigma is not None else None
    _check(lib().wsic_gather_features(
        _p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(sigma.data_ptr() if sigma is not None else 0),
        _rowmajor(sigma) if sigma is not None else n_in, _p(idx.data_ptr()), n_live, _p(Wl.data_ptr()), n_live,
        _p(Sl.data_ptr() if Sl is not None else 0), n_live, _stream(W)))
    return Wl, Sl


def scatter_codes(codes_live: torch.Tensor, pos: torch.Tensor, n_in: int) -> torch.Tensor:
    """Full code matrix: live columns from codes_live, dead columns 0."""
    _need_cuda(codes_live, pos)
    n_out = codes_live.shape[0]
    q = torch.empty((n_out, n_in), dtype=torch.int32, device=codes_live.device)
    _check(lib().wsic_scatter_codes(_p(codes_live.data_ptr()), n_out, _rowmajor(codes_live), _p(pos.data_ptr()),
                                    n_in, _p(q.data_ptr()), n_in, _stream(codes_live)))
    return q


def rans_encode(codes: torch.Tensor, lane_symbols: int = 256, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """Entropy-code the (contiguous) int32 codes: (container as a uint8 device tensor, bytes used)."""
    _need_cuda(codes)
    if codes.dtype != torch.int32 or not codes.is_contiguous():
        raise TypeError("codes must be contiguous int32")
    n = codes.numel()
    cap = int(lib().wsic_rans_bound(n, lane_symbols))
    if out is None or out.numel() < cap:
        out = torch.empty(cap, dtype=torch.uint8, device=codes.device)
    ws = ws if ws is not None else workspace(OP_RANS_ENC, lane_symbols, n, codes.device)
    nb = _sz(0)
    _check(lib().wsic_rans_encode(_p(codes.data_ptr()), n, lane_symbols, _p(out.data_ptr()), out.numel(),
                                  ctypes.byref(nb), *_ws_args(ws), _stream(codes)))
    return out, int(nb.value)


def rans_decode(blob: torch.Tensor, nbytes: int, n: int, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The n int32 codes of a container."""
    _need_cuda(blob)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=blob.device)
    ws = ws if ws is not None else workspace(OP_RANS_DEC, 1, 1, blob.device)
    _check(lib().wsic_rans_decode(_p(blob.data_ptr()), nbytes, _p(out.data_ptr()), n, *_ws_args(ws),
                                  _stream(blob)))
    return out


def rans_decode_dequant(blob: torch.Tensor, nbytes: int, n_out: int, n_in: int, U: torch.Tensor, c: float,
                        dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W_hat = c q / U_jj decoded straight from a container."""
    _need_cuda(blob, U)
    if out is None:
        out = torch.empty((n_out, n_in), dtype=dtype, device=blob.device)
    ws = ws if ws is not None else workspace(OP_RANS_DEC, 1, n_in, blob.device)
    _check(lib().wsic_rans_decode_dequant(_p(blob.data_ptr()), nbytes, n_out, n_in, _p(U.data_ptr()), _rowmajor(U),
                                          float(c), _p(out.data_ptr()), _dtype_code(out), *_ws_args(ws),
                                          _stream(blob)))
    return out


def distortion(W: torch.Tensor, codes: torch.Tensor, U: torch.Tensor, c: float,
               resid: Optional[torch.Tensor] = None, mode: str = "resid",
               w_hat_dtype: Optional[torch.dtype] = None, ws: Optional[torch.Tensor] = None):
    """Layer distortion tr((W - W_hat) Sigma (W - W_hat)^T); optionally W_hat."""
    _need_cuda(W, codes, U)
    n_out, n_in = W.shape
    w_hat = None
    wdt = F32
    if w_hat_dtype is not None:
        w_hat = torch.empty((n_out, n_in), dtype=w_hat_dtype, device=W.device)
        wdt = _dtype_code(w_hat)
    ws = ws if ws is not None else workspace(OP_DISTORTION, n_out, n_in, W.device)
    d = _d(0)
    _check(lib().wsic_distortion(
        _p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(codes.data_ptr()), _rowmajor(codes),
        _p(U.data_ptr()), _rowmajor(U), float(c), _p(resid.data_ptr() if resid is not None else 0),
        _rowmajor(resid) if resid is not None else n_in, D_DIRECT if mode == "direct" else D_RESID,
        ctypes.byref(d), _p(w_hat.data_ptr() if w_hat is not None else 0), wdt,
        _rowmajor(w_hat) if w_hat is not None else n_in, *_ws_args(ws), _stream(W)))
    return d.value, w_hat


def distortion_noalloc(W: torch.Tensor, codes: torch.Tensor, U: torch.Tensor, c: float,
                       resid: Optional[torch.Tensor] = None, mode: str = "resid",
                       w_hat: Optional[torch.Tensor] = None) -> float:
    """wsic_distortion_noalloc: the same distortion with the library's static scratch (no
    workspace); `w_hat` (optional) is a caller-allocated output."""
    _need_cuda(W, codes, U)
    n_out, n_in = W.shape
    d = _d(0)
    _check(lib().wsic_distortion_noalloc(
        _p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(codes.data_ptr()), _rowmajor(codes),
        _p(U.data_ptr()), _rowmajor(U), float(c), _p(resid.data_ptr() if resid is not None else 0),
        _rowmajor(resid) if resid is not None else n_in, D_DIRECT if mode == "direct" else D_RESID,
        ctypes.byref(d), _p(w_hat.data_ptr() if w_hat is not None else 0),
        _dtype_code(w_hat) if w_hat is not None else F32, _rowmajor(w_hat) if w_hat is not None else n_in,
        _stream(W)))
    return d.value


# ------------------------------------------------------------------------------ SoftWater
def softmax_curvature(X: torch.Tensor, W: torch.Tensor, smoothing: float = 0.0,
                      lam: Optional[torch.Tensor] = None, alpha: Optional[float] = None,
                      beta: float = 0.0, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lambda <- beta*lambda + alpha * sum over rows of X of p~(1 - p~), p~ the smoothed softmax
    of W x (alpha defaults to 1/rows: the mean over this chunk)."""
    _need_cuda(X, W)
    if X.dtype != W.dtype:
        raise TypeError("X and W must have the same dtype")
    rows, n = X.shape
    K = W.shape[0]
    if W.shape[1] != n:
        raise ValueError("W must have as many columns as X")
    if lam is None:
        lam = torch.zeros(K, dtype=torch.float64, device=X.device)
    ws = ws if ws is not None else workspace(OP_CURVATURE, rows, K, X.device)
    a = 1.0 / rows if alpha is None else float(alpha)
    _check(lib().wsic_softmax_curvature(_p(X.data_ptr()), _dtype_code(X), rows, n, _rowmajor(X), _p(W.data_ptr()),
                                        K, _rowmajor(W), float(smoothing), a, float(beta), _p(lam.data_ptr()),
                                        *_ws_args(ws), _stream(X)))
    return lam


def softmax_curvature_chunks(chunks: Sequence[torch.Tensor], W: torch.Tensor, smoothing: float = 0.0,
                             ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Class curvatures over streamed row chunks (the mean over all rows)."""
    n_total = sum(int(c.shape[0]) for c in chunks)
    lam = None
    for i, c in enumerate(chunks):
        if ws is None or ws.numel() < workspace_bytes(OP_CURVATURE, c.shape[0], W.shape[0]):
            ws = workspace(OP_CURVATURE, c.shape[0], W.shape[0], c.device)
        lam = softmax_curvature(c, W, smoothing, lam, alpha=1.0 / n_total, beta=0.0 if i == 0 else 1.0, ws=ws)
    return lam


def softwater_waterfill(W: torch.Tensor, U: torch.Tensor, lam: torch.Tensor, target_bits: float, *,
                        mode: str = "auto", rate_tol: float = 8e-5, bracket_log2: float = 2.0 ** -20,
                        max_passes: int = 64, c_init: float = 0.0, want_resid: bool = True,
                        codes: Optional[torch.Tensor] = None, resid: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """Waterfilling on the class-aware grids c / (sqrt(lam_k) U_jj)."""
    _need_cuda(W, U, lam)
    n_out, n_in = W.shape
    if lam.dtype != torch.float64 or lam.numel() != n_out:
        raise ValueError("lam must be float64 with one entry per row of W")
    if codes is None:
        codes = torch.empty((n_out, n_in), dtype=torch.int32, device=W.device)
    if want_resid and resid is None:
        resid = torch.empty((n_out, n_in), dtype=torch.float32, device=W.device)
    ws = ws if ws is not None else workspace(OP_SOFTWATER, n_out, n_in, W.device)
    opts = WfOpts(rate_tol, bracket_log2, max_passes, _MODES[mode], c_init, RATE_POOLED, 0)
    c_out, rate_out, passes = _d(0), _d(0), ctypes.c_int32(0)
    _check(lib().wsic_softwater_waterfill(
        _p(W.data_ptr()), _dtype_code(W), n_out, n_in, _rowmajor(W), _p(U.data_ptr()), _rowmajor(U),
        _p(lam.data_ptr()), float(target_bits), ctypes.byref(opts), ctypes.byref(c_out), ctypes.byref(rate_out),
        ctypes.byref(passes), _p(codes.data_ptr()), _rowmajor(codes),
        _p(resid.data_ptr() if resid is not None else 0), _rowmajor(resid) if resid is not None else n_in,
        *_ws_args(ws), _stream(W)))
    return {"c": c_out.value, "rate": rate_out.value, "passes": int(passes.value), "codes": codes,
            "resid": resid}


def softwater_distortion(codes: torch.Tensor, U: torch.Tensor, c: float, lam: torch.Tensor,
                         resid: torch.Tensor, w_hat_dtype: Optional[torch.dtype] = None,
                         ws: Optional[torch.Tensor] = None):
    """Second-order KL estimate 1/2 sum_k lam_k e_k Sigma e_k^T from the residuals; optionally W_hat."""
    _need_cuda(codes, U, lam, resid)
    n_out, n_in = codes.shape
    w_hat = None
    wdt = F32
    if w_hat_dtype is not None:
        w_hat = torch.empty((n_out, n_in), dtype=w_hat_dtype, device=codes.device)
        wdt = _dtype_code(w_hat)
    ws = ws if ws is not None else workspace(OP_SOFTWATER_DIST, n_out, n_in, codes.device)
    d = _d(0)
    _check(lib().wsic_softwater_distortion(
        _p(codes.data_ptr()), n_out, n_in, _rowmajor(codes), _p(U.data_ptr()), _rowmajor(U), float(c),
        _p(lam.data_ptr()), _p(resid.data_ptr()), _rowmajor(resid), ctypes.byref(d),
        _p(w_hat.data_ptr() if w_hat is not None else 0), wdt, _rowmajor(w_hat) if w_hat is not None else n_in,
        *_ws_args(ws), _stream(codes)))
    return d.value, w_hat


# ------------------------------------------------------------------------------ diagnostic switches
def debug_set(knob: str, value: float) -> None:
    """Select an alternative kernel path (same results) for tests; see wsic_debug_set."""
    _check(lib().wsic_debug_set(DEBUG_KNOBS[knob], float(value)))


def debug_get(knob: str) -> float:
    v = _d(0)
    _check(lib().wsic_debug_get(DEBUG_KNOBS[knob], ctypes.byref(v)))
    return v.value


def debug_reset() -> None:
    lib().wsic_debug_reset()


class debug:
    """Context manager: `with debug(guard_scale=3e4): ...` sets the switches and restores every
    default on exit."""

    def __init__(self, **knobs: float):
        self.knobs = knobs

    def __enter__(self):
        for k, v in self.knobs.items():
            debug_set(k, v)
        return self

    def __exit__(self, *exc):
        debug_reset()
        return False


# ------------------------------------------------------------------------------ kernel timing
def profile_enable(on: bool = True) -> None:
    _check(lib().wsic_profile_enable(1 if on else 0))


def profile_select(families: Optional[Sequence[str]] = None) -> None:
    """Time only these kernel families (None: all)."""
    arg = None if not families else ",".join(families).encode()
    _check(lib().wsic_profile_select(arg))


def profile_reset() -> None:
    _check(lib().wsic_profile_reset())


def profile_read(name: str) -> Dict[str, float]:
    n, ms, work = _i64(0), _d(0), _d(0)
    _check(lib().wsic_profile_read(name.encode(), ctypes.byref(n), ctypes.byref(ms), ctypes.byref(work)))
    return {"launches": int(n.value), "ms": ms.value, "work": work.value}


def profile_names() -> List[str]:
    buf = ctypes.create_string_buffer(4096)
    _check(lib().wsic_profile_names(buf, 4096))
    s = buf.value.decode()
    return [x for x in s.split(",") if x]


# ------------------------------------------------------------------------------ whole layer
def quantize_layer(W: torch.Tensor, x_chunks: Sequence[torch.Tensor], target_bits: float,
                   **wf_kw) -> Dict[str, object]:
    """Covariance -> Cholesky -> waterfill -> entropy -> distortion, all on the device."""
    sigma = covariance_chunks(x_chunks)
    U, _ = cholesky(sigma)
    wf = waterfill(W, U, target_bits, **wf_kw)
    h, nsym = entropy(wf["codes"])
    D, _ = distortion(W, wf["codes"], U, wf["c"], resid=wf["resid"])
    out = dict(wf)
    out.update({"U": U, "entropy": h, "n_symbols": nsym, "D": D})
    return out


def bf16_from_bits(bits, device) -> torch.Tensor:
    """uint16 numpy bf16 bit patterns -> device bfloat16 tensor (bit-exact)."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)

