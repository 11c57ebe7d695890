"""Host-side checks of libbsq.so (no GPU needed): the library loads, exports
every function include/bsq.h declares, and rejects invalid arguments on the
host before anything is enqueued (the pointers below are never dereferenced:
every call fails its host checks first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsq.h")


@pytest.fixture(scope="module")
def bsq():
    import block_scaled_precision_bsq_amd as b
    return b


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("bsq_quantize_nvfp4v", "bsq_quantize_mxfp8", "bsq_grouped_gemm_fwd", "bsq_grouped_gemm_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(bsq):
    lib = ctypes.CDLL(bsq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_helpers(bsq):
    assert bsq.ABI_VERSION == 5
    assert bsq.bsq_colwise_padded_cols(32, 32768) == 128 * (32 + 256)
    assert bsq.bsq_colwise_padded_cols(3, 0) == 384
    assert bsq.bsq_colwise_padded_cols(2, 129) == 128 * (2 + 2)
    assert bsq.bsq_colwise_padded_cols(2, 33) == 128 * (2 + 1)
    assert bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_FWD, 0, 1, 64, 64) == 0
    assert bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_FWD, 32, 1, 64, 64) % 256 == 0
    assert bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_BWD, 32, 1, 64, 64) > bsq.bsq_workspace_size(
        bsq.BSQ_OP_GEMM_FWD, 32, 1, 64, 64)
    assert bsq.bsq_workspace_size(7, 32, 1, 64, 64) == 0
    for s in range(5):
        assert bsq._lib.bsq_status_string(s)


FAKE = ctypes.c_void_p(0x100000)  # 256-byte aligned, never dereferenced


def test_quantize_host_checks(bsq):
    L = bsq._lib
    q = L.bsq_quantize_nvfp4v
    assert q(FAKE, 4, 15, 16, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_UNSUPPORTED   # cols % 16
    assert q(FAKE, 4, 32, 16, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG   # ld < cols
    assert q(None, 4, 32, 32, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG   # null input
    assert q(FAKE, -1, 32, 32, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG
    assert q(ctypes.c_void_p(0x100002), 4, 32, 32, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_UNSUPPORTED
    assert q(FAKE, 0, 32, 32, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_OK                # nothing to do
    assert q(FAKE, 4, 16400, 16400, None, 0, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_UNSUPPORTED
    m = L.bsq_quantize_mxfp8
    assert m(FAKE, 4, 48, 48, bsq.BSQ_ROWWISE, None, 0, FAKE, FAKE, None) == bsq.BSQ_ERR_UNSUPPORTED
    assert m(FAKE, 4, 64, 64, 5, None, 0, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG
    assert m(FAKE, 4, 64, 64, bsq.BSQ_COLWISE_T, None, 1, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG
    assert m(FAKE, 4, 60, 64, bsq.BSQ_COLWISE_T, FAKE, 1, FAKE, FAKE, None) == bsq.BSQ_ERR_UNSUPPORTED
    d = L.bsq_quantize_mxfp8_dual
    assert d(FAKE, 4, 64, 64, None, 1, FAKE, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG  # no offsets
    assert d(FAKE, 4, 64, 64, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG  # no groups
    assert d(FAKE, 4, 48, 48, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_UNSUPPORTED  # cols % 32
    assert d(FAKE, 4, 64, 32, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG  # ld < cols
    assert d(FAKE, 4, 64, 64, FAKE, 1, None, FAKE, FAKE, FAKE, None) == bsq.BSQ_ERR_INVALID_ARG  # null output
    assert d(FAKE, 0, 64, 64, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None) == bsq.BSQ_OK              # nothing to do


def test_gemm_host_checks(bsq):
    L = bsq._lib
    f = L.bsq_grouped_gemm_fwd
    need = bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_FWD, 4, 64, 64, 128)
    args = lambda n, k, ws, E=4, dt=bsq.BSQ_BF16: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, E, 64, n, k, FAKE,
                                                     dt, FAKE, ws, None)
    assert f(*args(64, 96, need)) == bsq.BSQ_ERR_UNSUPPORTED          # k % 64
    assert f(*args(60, 128, need)) == bsq.BSQ_ERR_UNSUPPORTED         # n % 8
    assert f(*args(64, 128, need - 1)) == bsq.BSQ_ERR_WORKSPACE_TOO_SMALL
    assert f(*args(64, 128, need, E=0)) == bsq.BSQ_ERR_INVALID_ARG
    assert f(*args(64, 128, need, dt=9)) == bsq.BSQ_ERR_INVALID_ARG
    b = L.bsq_grouped_gemm_bwd
    needb = bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_BWD, 4, 64, 64, 128)
    bargs = lambda n, k, flags, ws: (FAKE,) * 9 + (4, 64, n, k, FAKE, bsq.BSQ_BF16, FAKE, bsq.BSQ_BF16, flags,
                                                   FAKE, ws, None)
    assert b(*bargs(64, 128, 0, needb)) == bsq.BSQ_ERR_INVALID_ARG     # no GEMM requested
    assert b(*bargs(64, 128, 4, needb)) == bsq.BSQ_ERR_INVALID_ARG     # unknown flag
    assert b(*bargs(96, 128, 3, needb)) == bsq.BSQ_ERR_UNSUPPORTED     # n % 64
    assert b(*bargs(64, 128, 3, needb - 1)) == bsq.BSQ_ERR_WORKSPACE_TOO_SMALL
    w = L.bsq_grouped_gemm_w4a16
    wargs = lambda n, k, ws, rs=FAKE: (FAKE, FAKE, FAKE, rs, FAKE, 4, 64, n, k, FAKE, bsq.BSQ_BF16, FAKE, ws, None)
    assert w(*wargs(64, 96, need)) == bsq.BSQ_ERR_UNSUPPORTED          # k % 64
    assert w(*wargs(96, 128, need)) == bsq.BSQ_ERR_UNSUPPORTED         # n % 64
    assert w(*wargs(64, 128, need, rs=None)) == bsq.BSQ_ERR_INVALID_ARG  # no row scales
    assert w(*wargs(64, 128, need - 1)) == bsq.BSQ_ERR_WORKSPACE_TOO_SMALL


def test_product_path_has_no_oracle_or_fallback():
    """The library package never imports the oracle and has no CPU path."""
    pkg = os.path.join(ROOT, "block_scaled_precision_bsq_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn


def test_noalloc_host_checks(bsq):
    """The allocation-free forward GEMM rejects expert counts its device array
    cannot plan for, before touching the device."""
    f = bsq._lib.bsq_grouped_gemm_fwd_noalloc
    args = lambda E: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, E, 64, 64, 128, FAKE, bsq.BSQ_BF16, None)
    assert f(*args(4097)) == bsq.BSQ_ERR_UNSUPPORTED
    assert f(*args(0)) == bsq.BSQ_ERR_INVALID_ARG
    assert f(*args(-3)) == bsq.BSQ_ERR_INVALID_ARG


def test_gemm_swiglu_host_checks(bsq):
    """The fused gate/up + SwiGLU GEMM needs inter % 128 == 0 (a 256-column
    tile holds 128 gate and the matching 128 up columns) and a valid H pitch."""
    f = bsq._lib.bsq_grouped_gemm_fwd_swiglu
    need = bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_FWD, 4, 64, 256, 128)
    args = lambda inter, k, ldh, ws=need, E=4, h=FAKE: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, E, 64, inter, k,
                                                        h, ldh, FAKE, ws, None)
    assert f(*args(64, 128, 64)) == bsq.BSQ_ERR_UNSUPPORTED      # inter % 128
    assert f(*args(128, 96, 128)) == bsq.BSQ_ERR_UNSUPPORTED     # k % 64
    assert f(*args(128, 128, 100)) == bsq.BSQ_ERR_INVALID_ARG    # ld_h < inter
    assert f(*args(128, 128, 132)) == bsq.BSQ_ERR_UNSUPPORTED    # ld_h % 8
    assert f(*args(128, 128, 128, h=None)) == bsq.BSQ_ERR_INVALID_ARG
    assert f(*args(128, 128, 128, E=0)) == bsq.BSQ_ERR_INVALID_ARG
    assert f(*args(128, 128, 128, ws=need - 1)) == bsq.BSQ_ERR_WORKSPACE_TOO_SMALL
