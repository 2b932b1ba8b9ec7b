"""Host-side checks of libwsic that need no GPU: the library loads, exports every function
include/wsic.h declares, and its argument checks reject bad calls before any device work."""
import ctypes
import os
import subprocess
import sys

import pytest

from rate_allocated_weight_amd import _lib as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_declares_the_boundary():
    names = W.header_functions()
    for required in ("wsic_covariance", "wsic_cholesky", "wsic_waterfill", "wsic_sic_quantize",
                     "wsic_entropy", "wsic_distortion"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = W.lib()
    missing = [n for n in W.header_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding knows every declared function too
    assert set(W.header_functions()) <= set(W._SIGS)


def test_version_and_status_strings():
    lib = W.lib()
    assert lib.wsic_version() == 100
    for code, name in [(0, "WSIC_OK"), (-1, "WSIC_E_INVAL"), (-2, "WSIC_E_NOT_PD"),
                       (-3, "WSIC_E_NONFINITE"), (-4, "WSIC_E_NO_BRACKET"), (-5, "WSIC_E_RANGE"),
                       (-6, "WSIC_E_WORKSPACE"), (-7, "WSIC_E_HIP")]:
        assert lib.wsic_status_str(code).decode() == name


def test_workspace_sizes():
    n_out, n_in = 4096, 4096
    sic = W.workspace_bytes(W.OP_SIC, n_out, n_in)
    assert sic >= 2 * 8 * n_out * n_in  # Y and G in fp64
    wf = W.workspace_bytes(W.OP_WATERFILL, n_out, n_in)
    assert wf >= sic + 8 * n_out * n_in  # plus a second code and residual buffer
    assert W.workspace_bytes(W.OP_ENTROPY, 10, 10) > 4 * (1 << 20)
    assert W.workspace_bytes(W.OP_COVARIANCE, 0, 64) > 0
    assert W.workspace_bytes(99, 10, 10) == 0
    assert W.workspace_bytes(W.OP_SIC, 0, 10) == 0
    for op in range(6):
        assert W.workspace_bytes(op, 100, 300) % 256 == 0


def test_argument_checks_return_before_device_work():
    lib = W.lib()
    p = ctypes.c_void_p
    fake = p(0x1000)  # never dereferenced: every call below fails validation first
    ws = p(0x100000)
    c_out, r_out, passes = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    # null W
    st = lib.wsic_sic_quantize(None, W.BF16, 4, 4, 4, fake, 4, 1.0, fake, 4, None, 4, ws, 1 << 30, None)
    assert st == W.E_INVAL and b"null" in lib.wsic_last_error()
    # ld too small
    st = lib.wsic_sic_quantize(fake, W.BF16, 4, 8, 4, fake, 8, 1.0, fake, 8, None, 8, ws, 1 << 30, None)
    assert st == W.E_INVAL
    # bad dtype
    st = lib.wsic_sic_quantize(fake, 7, 4, 4, 4, fake, 4, 1.0, fake, 4, None, 4, ws, 1 << 30, None)
    assert st == W.E_INVAL
    # non-positive grid scale
    st = lib.wsic_sic_quantize(fake, W.F32, 4, 4, 4, fake, 4, 0.0, fake, 4, None, 4, ws, 1 << 30, None)
    assert st == W.E_INVAL
    # workspace too small
    st = lib.wsic_sic_quantize(fake, W.F32, 4, 4, 4, fake, 4, 1.0, fake, 4, None, 4, ws, 16, None)
    assert st == W.E_WORKSPACE and b"workspace" in lib.wsic_last_error()
    # misaligned workspace
    st = lib.wsic_sic_quantize(fake, W.F32, 4, 4, 4, fake, 4, 1.0, fake, 4, None, 4, p(0x100010), 1 << 30, None)
    assert st == W.E_INVAL
    # target rate must be positive; bad controller mode
    st = lib.wsic_waterfill(fake, W.F32, 4, 4, 4, fake, 4, 0.0, None, ctypes.byref(c_out), ctypes.byref(r_out),
                            ctypes.byref(passes), fake, 4, None, 4, ws, 1 << 30, None)
    assert st == W.E_INVAL
    opts = W.WfOpts(1e-5, 1e-6, 10, 9, 0.0)
    st = lib.wsic_waterfill(fake, W.F32, 4, 4, 4, fake, 4, 2.0, ctypes.byref(opts), ctypes.byref(c_out),
                            ctypes.byref(r_out), ctypes.byref(passes), fake, 4, None, 4, ws, 1 << 30, None)
    assert st == W.E_INVAL and b"mode" in lib.wsic_last_error()
    # covariance / cholesky / entropy / distortion shapes
    assert lib.wsic_covariance(fake, W.BF16, 0, 4, 4, 1.0, 0.0, fake, 4, ws, 1 << 20, None) == W.E_INVAL
    info = ctypes.c_int64(5)
    assert lib.wsic_cholesky(fake, 8, 4, ctypes.byref(info), ws, 1 << 20, None) == W.E_INVAL
    h, ns = ctypes.c_double(), ctypes.c_int64()
    assert lib.wsic_entropy(None, 4, 4, 4, ctypes.byref(h), ctypes.byref(ns), ws, 1 << 30, None) == W.E_INVAL
    d = ctypes.c_double()
    # resid mode without residuals
    st = lib.wsic_distortion(fake, W.F32, 4, 4, 4, fake, 4, fake, 4, 1.0, None, 4, W.D_RESID, ctypes.byref(d),
                             None, W.F32, 4, ws, 1 << 30, None)
    assert st == W.E_INVAL
    # an error message does not leak into the next successful query
    assert lib.wsic_version() == 100


def test_product_path_has_no_oracle_dependency():
    """Nothing in the package imports the oracle, and the package refuses to run without
    its HIP library (no CPU fallback)."""
    pkg = os.path.join(ROOT, "rate_allocated_weight_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
    code = ("import rate_allocated_weight_amd._lib as L; L.LIB_PATH = '/nonexistent/libwsic.so'; "
            "L._LIB = None\n"
            "try:\n    L.lib()\nexcept ImportError as e:\n    print('refused')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "refused" in out.stdout, out.stderr


def test_debug_switches_are_explicit_and_bounded():
    """Alternative kernel paths are chosen only through wsic_debug_set (no environment
    variable), and no value may weaken the int8 product's exact re-check."""
    W.debug_reset()
    assert W.debug_get("guard_scale") == 1.0
    assert W.debug_get("super_blocks") == 1.0 and W.debug_get("fp64_product") == 0.0
    for bad in (0.5, 0.0, -3.0, float("nan"), float("inf")):
        with pytest.raises(W.WsicError) as ei:
            W.debug_set("guard_scale", bad)
        assert ei.value.status == W.E_INVAL
        assert W.debug_get("guard_scale") == 1.0
    with W.debug(guard_scale=3e4, super_blocks=0):
        assert W.debug_get("guard_scale") == 3e4 and W.debug_get("super_blocks") == 0.0
    assert W.debug_get("guard_scale") == 1.0 and W.debug_get("super_blocks") == 1.0
    assert W.lib().wsic_debug_set(99, 1.0) == W.E_INVAL
    src = open(os.path.join(ROOT, "rate_allocated_weight_amd", "csrc", "wsic_api.hip")).read()
    assert "getenv" not in src
