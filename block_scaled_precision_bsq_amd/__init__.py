"""Python binding of libbsq.so: block-scaled MoE expert grouped GEMM on MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/bsq.h``: every
function here has the C entry point's name, checks tensor dtypes, shapes and
devices, passes raw device pointers plus torch's current HIP stream, and turns
a non-OK status into ``RuntimeError``.  All arithmetic runs in the HIP kernels;
torch only provides device memory and streams.  There is no CPU fallback:
importing this package fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python block_scaled_precision_bsq_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32
INT = ctypes.c_int

BSQ_OK, BSQ_ERR_INVALID_ARG, BSQ_ERR_UNSUPPORTED, BSQ_ERR_WORKSPACE_TOO_SMALL, BSQ_ERR_HIP = range(5)
BSQ_BF16, BSQ_F32 = 0, 1
BSQ_ROWWISE, BSQ_COLWISE_T = 0, 1
BSQ_DGRAD, BSQ_WGRAD = 1, 2
BSQ_OP_GEMM_FWD, BSQ_OP_GEMM_BWD = 0, 1

_SIGS = {
    "bsq_quantize_nvfp4v": ([P, I64, I64, I64, P, I32, P, P, P, P], INT),
    "bsq_swiglu_quantize_nvfp4v": ([P, I64, I64, I64, P, I64, P, P, P, P], INT),
    "bsq_quantize_mxfp8_gather": ([P, I64, I64, I64, P, I64, P, P, P], INT),
    "bsq_debug_quantize_nvfp4v_fastdiv": ([P, I64, I64, I64, P, P, P, P], INT),
    "bsq_quantize_mxfp8": ([P, I64, I64, I64, INT, P, I32, P, P, P], INT),
    "bsq_quantize_mxfp8_dual": ([P, I64, I64, I64, P, I32, P, P, P, P, P], INT),
    "bsq_grouped_gemm_fwd": ([P, P, P, P, P, P, P, I32, I64, I64, I64, P, INT, P, ctypes.c_size_t, P], INT),
    "bsq_grouped_gemm_fwd_swiglu": ([P, P, P, P, P, P, P, I32, I64, I64, I64, P, I64, P, ctypes.c_size_t, P], INT),
    "bsq_grouped_gemm_fwd_noalloc": ([P, P, P, P, P, P, P, I32, I64, I64, I64, P, INT, P], INT),
    "bsq_grouped_gemm_bwd": ([P, P, P, P, P, P, P, P, P, I32, I64, I64, I64, P, INT, P, INT, ctypes.c_uint, P,
                              ctypes.c_size_t, P], INT),
    "bsq_grouped_gemm_fwd_mxfp8": ([P, P, P, P, P, I32, I64, I64, I64, P, INT, P, ctypes.c_size_t, P], INT),
    "bsq_grouped_gemm_bf16": ([P, P, P, I32, I64, I64, I64, P, INT, P, ctypes.c_size_t, P], INT),
    "bsq_grouped_gemm_w4a16": ([P, P, P, P, P, I32, I64, I64, I64, P, INT, P, ctypes.c_size_t, P], INT),
    "bsq_workspace_size": ([INT, I32, I64, I64, I64], ctypes.c_size_t),
    "bsq_colwise_padded_cols": ([I32, I64], I64),
    "bsq_status_string": ([INT], ctypes.c_char_p),
    "bsq_abi_version": ([], INT),
    "bsq_debug_status": ([P, P, ctypes.POINTER(I32)], INT),
    "bsq_debug_encode_e2m1": ([P, P, I64, P], INT),
    "bsq_debug_encode_e4m3": ([P, P, I64, P], INT),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

ABI_VERSION = _lib.bsq_abi_version()


class BsqError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {_lib.bsq_status_string(status).decode()} (status {status})")
        self.status = status


def _check(fn, status):
    if status != BSQ_OK:
        raise BsqError(fn, status)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(stream, shape, dtype, device):
    """torch.empty on the caching allocator's pool of ``stream`` when one is
    given: a block freed here (the workspace) or later (an output) is then
    reused only in ``stream``'s order, never while its kernels still run."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, name, dtypes):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _rows_ld(x):
    if x.dim() != 2:
        raise ValueError("x must be a 2-D matrix")
    rows, cols = x.shape
    if rows == 0 or cols == 0:
        return rows, cols, cols
    if x.stride(1) != 1 and cols > 1:
        raise ValueError("x must be row-major (unit column stride)")
    return rows, cols, x.stride(0) if rows > 1 else cols


def bsq_workspace_size(op, num_experts, m_total, n, k):
    return int(_lib.bsq_workspace_size(op, num_experts, m_total, n, k))


def bsq_colwise_padded_cols(num_groups, rows):
    return int(_lib.bsq_colwise_padded_cols(num_groups, rows))


def bsq_quantize_nvfp4v(x, codes=None, bscale=None, rscale=None, offsets=None, stream=None):
    """NVFP4-variant quantization of each row of bf16 ``x`` [rows, cols].
    Returns (codes u8 [rows, cols/2], bscale u8 [rows, cols/16], rscale f32 [rows])."""
    _dev(x, "x", _BF16)
    rows, cols, ld = _rows_ld(x)
    dev = x.device
    codes = _empty(stream, (rows, cols // 2), dtype=torch.uint8, device=dev) if codes is None else codes
    bscale = _empty(stream, (rows, cols // 16), dtype=torch.uint8, device=dev) if bscale is None else bscale
    rscale = _empty(stream, (rows,), dtype=torch.float32, device=dev) if rscale is None else rscale
    for t, nm, shape in ((codes, "codes", (rows, cols // 2)), (bscale, "bscale", (rows, cols // 16)),
                         (rscale, "rscale", (rows,))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
    ng = 0 if offsets is None else offsets.numel() - 1
    _check("bsq_quantize_nvfp4v",
           _lib.bsq_quantize_nvfp4v(_ptr(x), rows, cols, ld, _ptr(offsets), ng, _ptr(codes), _ptr(bscale),
                                    _ptr(rscale), _stream(stream)))
    return codes, bscale, rscale


def bsq_debug_quantize_nvfp4v_fastdiv(x, stream=None):
    """Ablation: bsq_quantize_nvfp4v with fast approximate divides (reciprocal
    approximation times numerator).  Returns (codes, bscale, rscale)."""
    _dev(x, "x", _BF16)
    rows, cols, ld = _rows_ld(x)
    dev = x.device
    codes = _empty(stream, (rows, cols // 2), dtype=torch.uint8, device=dev)
    bscale = _empty(stream, (rows, cols // 16), dtype=torch.uint8, device=dev)
    rscale = _empty(stream, (rows,), dtype=torch.float32, device=dev)
    _check("bsq_debug_quantize_nvfp4v_fastdiv",
           _lib.bsq_debug_quantize_nvfp4v_fastdiv(_ptr(x), rows, cols, ld, _ptr(codes), _ptr(bscale), _ptr(rscale),
                                                  _stream(stream)))
    return codes, bscale, rscale


def bsq_quantize_mxfp8_gather(x, row_index, codes=None, scale=None, stream=None):
    """MXFP8 ROWWISE quantization of the rows ``x[row_index]`` (int32 device
    indices; out-of-range indices give zero rows) in one pass.
    Returns (codes [rows, cols], scale [cols/32, rows])."""
    _dev(x, "x", _BF16)
    _dev(row_index, "row_index", (torch.int32,))
    src_rows, cols, ld = _rows_ld(x)
    rows = row_index.numel()
    dev = x.device
    codes = _empty(stream, (rows, cols), dtype=torch.uint8, device=dev) if codes is None else codes
    scale = _empty(stream, (cols // 32, rows), dtype=torch.uint8, device=dev) if scale is None else scale
    for t, nm, shape in ((codes, "codes", (rows, cols)), (scale, "scale", (cols // 32, rows))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
    _check("bsq_quantize_mxfp8_gather",
           _lib.bsq_quantize_mxfp8_gather(_ptr(x), src_rows, cols, ld, _ptr(row_index), rows, _ptr(codes),
                                          _ptr(scale), _stream(stream)))
    return codes, scale


def bsq_swiglu_quantize_nvfp4v(gu, h=None, write_h=True, codes=None, bscale=None, rscale=None, stream=None):
    """SwiGLU of bf16 ``gu`` [rows, 2*inter] ([gate | up] per row) fused with the
    NVFP4-variant quantization of H = bf16(silu(gate) * up).
    Returns (h bf16 [rows, inter] or None, codes u8 [rows, inter/2],
    bscale u8 [rows, inter/16], rscale f32 [rows])."""
    _dev(gu, "gu", _BF16)
    rows, cols2, ld = _rows_ld(gu)
    if cols2 % 2:
        raise ValueError("gu must have an even number of columns ([gate | up])")
    inter = cols2 // 2
    dev = gu.device
    if write_h and h is None:
        h = _empty(stream, (rows, inter), dtype=torch.bfloat16, device=dev)
    if h is not None:
        _dev(h, "h", _BF16)
        if tuple(h.shape) != (rows, inter) or (rows > 1 and h.stride(1) != 1):
            raise ValueError(f"h must be row-major with shape {(rows, inter)}")
    ldh = 0 if h is None else (h.stride(0) if rows > 1 else inter)
    codes = _empty(stream, (rows, inter // 2), dtype=torch.uint8, device=dev) if codes is None else codes
    bscale = _empty(stream, (rows, inter // 16), dtype=torch.uint8, device=dev) if bscale is None else bscale
    rscale = _empty(stream, (rows,), dtype=torch.float32, device=dev) if rscale is None else rscale
    for t, nm, shape in ((codes, "codes", (rows, inter // 2)), (bscale, "bscale", (rows, inter // 16)),
                         (rscale, "rscale", (rows,))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
    _check("bsq_swiglu_quantize_nvfp4v",
           _lib.bsq_swiglu_quantize_nvfp4v(_ptr(gu), rows, inter, ld, _ptr(h), ldh, _ptr(codes), _ptr(bscale),
                                           _ptr(rscale), _stream(stream)))
    return h, codes, bscale, rscale


def bsq_quantize_mxfp8(x, axis=BSQ_ROWWISE, offsets=None, codes=None, scale=None, stream=None):
    """MXFP8 quantization of bf16 ``x`` [rows, cols]; scales are block-major.
    ROWWISE: (codes [rows, cols], scale [cols/32, rows]).
    COLWISE_T (needs int32 device ``offsets``): (codes [cols, P], scale [P/32, cols])."""
    _dev(x, "x", _BF16)
    rows, cols, ld = _rows_ld(x)
    dev = x.device
    if axis == BSQ_ROWWISE:
        shapes = ((rows, cols), (cols // 32, rows))
        ng = 0
    else:
        if offsets is None:
            raise ValueError("COLWISE_T needs offsets")
        _dev(offsets, "offsets", (torch.int32,))
        ng = offsets.numel() - 1
        Pc = bsq_colwise_padded_cols(ng, rows)
        shapes = ((cols, Pc), (Pc // 32, cols))
    codes = _empty(stream, shapes[0], dtype=torch.uint8, device=dev) if codes is None else codes
    scale = _empty(stream, shapes[1], dtype=torch.uint8, device=dev) if scale is None else scale
    for t, nm, shape in ((codes, "codes", shapes[0]), (scale, "scale", shapes[1])):
        if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
    _check("bsq_quantize_mxfp8",
           _lib.bsq_quantize_mxfp8(_ptr(x), rows, cols, ld, axis, _ptr(offsets), ng, _ptr(codes), _ptr(scale),
                                   _stream(stream)))
    return codes, scale


def bsq_quantize_mxfp8_dual(x, offsets, row=None, t=None, stream=None):
    """Both MXFP8 layouts of bf16 ``x`` [rows, cols] from one read: returns
    ((codes [rows, cols], scale [cols/32, rows]) as ROWWISE,
     (codes [cols, P], scale [P/32, cols]) as COLWISE_T with int32 ``offsets``)."""
    _dev(x, "x", _BF16)
    _dev(offsets, "offsets", (torch.int32,))
    rows, cols, ld = _rows_ld(x)
    dev = x.device
    ng = offsets.numel() - 1
    Pc = bsq_colwise_padded_cols(ng, rows)
    shapes = ((rows, cols), (cols // 32, rows), (cols, Pc), (Pc // 32, cols))
    rc, rs = (None, None) if row is None else row
    tc, ts = (None, None) if t is None else t
    outs = []
    for buf, nm, shape in ((rc, "row codes", shapes[0]), (rs, "row scale", shapes[1]),
                           (tc, "t codes", shapes[2]), (ts, "t scale", shapes[3])):
        buf = _empty(stream, shape, dtype=torch.uint8, device=dev) if buf is None else buf
        if tuple(buf.shape) != tuple(shape) or not buf.is_contiguous():
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
        outs.append(buf)
    _check("bsq_quantize_mxfp8_dual",
           _lib.bsq_quantize_mxfp8_dual(_ptr(x), rows, cols, ld, _ptr(offsets), ng, *[_ptr(o) for o in outs],
                                        _stream(stream)))
    return (outs[0], outs[1]), (outs[2], outs[3])


def _workspace(op, E, m_total, n, k, workspace, dev, stream=None):
    need = bsq_workspace_size(op, E, m_total, n, k)
    if workspace is None:
        workspace = _empty(stream, (need,), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    return workspace


def bsq_grouped_gemm_fwd(a_q, w_q, offsets, n, k, y_dtype=BSQ_BF16, y=None, workspace=None, stream=None):
    """Forward grouped GEMM.  a_q / w_q = (codes, bscale, rscale) of the
    expert-sorted activations [m_total, k] and of the weights [E*n, k]."""
    a_codes, a_bscale, a_rscale = a_q
    w_codes, w_bscale, w_rscale = w_q
    _dev(offsets, "offsets", (torch.int32,))
    E = offsets.numel() - 1
    m_total = a_codes.shape[0]
    if w_codes.shape[0] != E * n:
        raise ValueError("weights must hold num_experts * n rows")
    dev = a_codes.device
    if y is None:
        y = _empty(stream, (m_total, n), dtype=torch.float32 if y_dtype == BSQ_F32 else torch.bfloat16, device=dev)
    workspace = _workspace(BSQ_OP_GEMM_FWD, E, m_total, n, k, workspace, dev, stream)
    _check("bsq_grouped_gemm_fwd",
           _lib.bsq_grouped_gemm_fwd(_ptr(a_codes), _ptr(a_bscale), _ptr(a_rscale), _ptr(w_codes), _ptr(w_bscale),
                                     _ptr(w_rscale), _ptr(offsets), E, m_total, n, k, _ptr(y), y_dtype,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
    return y


def bsq_grouped_gemm_fwd_swiglu(a_q, w_q, offsets, inter, k, h=None, workspace=None, stream=None):
    """Gate/up grouped GEMM with the SwiGLU activation in its epilogue.
    a_q = NVFP4v (codes, bscale, rscale) of the expert-sorted activations
    [m_total, k]; w_q = NVFP4v of the gate/up weights [E*2*inter, k] ([gate;
    up] rows per expert).  Returns h bf16 [m_total, inter]; the gate/up output
    is never written."""
    a_codes, a_bscale, a_rscale = a_q
    w_codes, w_bscale, w_rscale = w_q
    _dev(offsets, "offsets", (torch.int32,))
    E = offsets.numel() - 1
    m_total = a_codes.shape[0]
    if w_codes.shape[0] != E * 2 * inter:
        raise ValueError("weights must hold num_experts * 2 * inter rows")
    dev = a_codes.device
    if h is None:
        h = _empty(stream, (m_total, inter), dtype=torch.bfloat16, device=dev)
    _dev(h, "h", _BF16)
    if tuple(h.shape) != (m_total, inter) or (m_total > 1 and h.stride(1) != 1):
        raise ValueError(f"h must be row-major with shape {(m_total, inter)}")
    ldh = h.stride(0) if m_total > 1 else inter
    workspace = _workspace(BSQ_OP_GEMM_FWD, E, m_total, 2 * inter, k, workspace, dev, stream)
    _check("bsq_grouped_gemm_fwd_swiglu",
           _lib.bsq_grouped_gemm_fwd_swiglu(_ptr(a_codes), _ptr(a_bscale), _ptr(a_rscale), _ptr(w_codes),
                                            _ptr(w_bscale), _ptr(w_rscale), _ptr(offsets), E, m_total, inter, k,
                                            _ptr(h), ldh, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))
    return h


def bsq_grouped_gemm_fwd_noalloc(a_q, w_q, offsets, n, k, y_dtype=BSQ_BF16, y=None, stream=None):
    """bsq_grouped_gemm_fwd with the planner workspace inside the library (no
    workspace argument; the library allocates nothing).  ``y`` is allocated
    here only when not given."""
    a_codes, a_bscale, a_rscale = a_q
    w_codes, w_bscale, w_rscale = w_q
    _dev(offsets, "offsets", (torch.int32,))
    E = offsets.numel() - 1
    m_total = a_codes.shape[0]
    if w_codes.shape[0] != E * n:
        raise ValueError("weights must hold num_experts * n rows")
    if y is None:
        y = _empty(stream, (m_total, n), dtype=torch.float32 if y_dtype == BSQ_F32 else torch.bfloat16,
                   device=a_codes.device)
    _check("bsq_grouped_gemm_fwd_noalloc",
           _lib.bsq_grouped_gemm_fwd_noalloc(_ptr(a_codes), _ptr(a_bscale), _ptr(a_rscale), _ptr(w_codes),
                                             _ptr(w_bscale), _ptr(w_rscale), _ptr(offsets), E, m_total, n, k, _ptr(y),
                                             y_dtype, _stream(stream)))
    return y


def bsq_grouped_gemm_fwd_mxfp8(x_q, w_q, offsets, n, k, y_dtype=BSQ_BF16, y=None, workspace=None, stream=None):
    """Forward grouped GEMM over MXFP8 operands.  x_q / w_q = ROWWISE (codes,
    scale) of the expert-sorted activations [m_total, k] and of the weights
    [E*n, k] (block-major scales)."""
    x_codes, x_scale = x_q
    w_codes, w_scale = w_q
    _dev(offsets, "offsets", (torch.int32,))
    E = offsets.numel() - 1
    m_total = x_codes.shape[0]
    if w_codes.shape[0] != E * n:
        raise ValueError("weights must hold num_experts * n rows")
    dev = x_codes.device
    if y is None:
        y = _empty(stream, (m_total, n), dtype=torch.float32 if y_dtype == BSQ_F32 else torch.bfloat16, device=dev)
    workspace = _workspace(BSQ_OP_GEMM_FWD, E, m_total, n, k, workspace, dev, stream)
    _check("bsq_grouped_gemm_fwd_mxfp8",
           _lib.bsq_grouped_gemm_fwd_mxfp8(_ptr(x_codes), _ptr(x_scale), _ptr(w_codes), _ptr(w_scale),
                                           _ptr(offsets), E, m_total, n, k, _ptr(y), y_dtype, _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def bsq_grouped_gemm_bf16(x, w, offsets, n, k, y_dtype=BSQ_BF16, y=None, workspace=None, stream=None):
    """bf16 baseline grouped GEMM: x [m_total, k] bf16, w [E*n, k] bf16."""
    _dev(x, "x", _BF16)
    _dev(w, "w", _BF16)
    _dev(offsets, "offsets", (torch.int32,))
    E = offsets.numel() - 1
    m_total = x.shape[0]
    for t, nm, shape in ((x, "x", (m_total, k)), (w, "w", (E * n, k))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
    dev = x.device
    if y is None:
        y = _empty(stream, (m_total, n), dtype=torch.float32 if y_dtype == BSQ_F32 else torch.bfloat16, device=dev)
    workspace = _workspace(BSQ_OP_GEMM_FWD, E, m_total, n, k, workspace, dev, stream)
    _check("bsq_grouped_gemm_bf16",
           _lib.bsq_grouped_gemm_bf16(_ptr(x), _ptr(w), _ptr(offsets), E, m_total, n, k, _ptr(y), y_dtype,
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))
    return y


def bsq_grouped_gemm_w4a16(x, w_q, offsets, n, k, y_dtype=BSQ_BF16, y=None, workspace=None, stream=None):
    """Frozen-expert GEMM: x [m_total, k] bf16 against packed weights
    w_q = (codes [E*n, k/2], bscale [E*n, k/16], rscale [E*n]) from
    bsq_quantize_nvfp4v, dequantized to bf16 inside the kernel."""
    _dev(x, "x", _BF16)
    _dev(offsets, "offsets", (torch.int32,))
    w_codes, w_bscale, w_rscale = w_q
    E = offsets.numel() - 1
    m_total = x.shape[0]
    for t, nm, shape, dt in ((x, "x", (m_total, k), None), (w_codes, "w codes", (E * n, k // 2), torch.uint8),
                             (w_bscale, "w bscale", (E * n, k // 16), torch.uint8),
                             (w_rscale, "w rscale", (E * n,), torch.float32)):
        if tuple(t.shape) != shape or not t.is_contiguous() or (dt is not None and t.dtype != dt):
            raise ValueError(f"{nm} must be contiguous with shape {shape}")
    dev = x.device
    if y is None:
        y = _empty(stream, (m_total, n), dtype=torch.float32 if y_dtype == BSQ_F32 else torch.bfloat16, device=dev)
    workspace = _workspace(BSQ_OP_GEMM_FWD, E, m_total, n, k, workspace, dev, stream)
    _check("bsq_grouped_gemm_w4a16",
           _lib.bsq_grouped_gemm_w4a16(_ptr(x), _ptr(w_codes), _ptr(w_bscale), _ptr(w_rscale), _ptr(offsets), E,
                                       m_total, n, k, _ptr(y), y_dtype, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def bsq_grouped_gemm_bwd(offsets, m_total, n, k, dy_q=None, wt_q=None, dyt_q=None, xt_q=None,
                         flags=BSQ_DGRAD | BSQ_WGRAD, dx_dtype=BSQ_BF16, dw_dtype=BSQ_BF16, dx=None, dw=None,
                         workspace=None, stream=None):
    """Backward grouped GEMMs.  dy_q = ROWWISE (codes, scale) of dY [m_total, n];
    wt_q = COLWISE_T of W [E*n, k] with offsets {0, n, 2n, ..}; dyt_q / xt_q =
    COLWISE_T of dY / X with ``offsets``.  Returns (dx, dw)."""
    _dev(offsets, "offsets", (torch.int32,))
    E = offsets.numel() - 1
    dev = offsets.device
    if flags & BSQ_DGRAD and dx is None and m_total > 0:
        dx = _empty(stream, (m_total, k), dtype=torch.float32 if dx_dtype == BSQ_F32 else torch.bfloat16, device=dev)
    if flags & BSQ_WGRAD and dw is None:
        dw = _empty(stream, (E, n, k), dtype=torch.float32 if dw_dtype == BSQ_F32 else torch.bfloat16, device=dev)
    workspace = _workspace(BSQ_OP_GEMM_BWD, E, m_total, n, k, workspace, dev, stream)
    dy_q = dy_q or (None, None)
    wt_q = wt_q or (None, None)
    dyt_q = dyt_q or (None, None)
    xt_q = xt_q or (None, None)
    _check("bsq_grouped_gemm_bwd",
           _lib.bsq_grouped_gemm_bwd(_ptr(dy_q[0]), _ptr(dy_q[1]), _ptr(wt_q[0]), _ptr(wt_q[1]), _ptr(dyt_q[0]),
                                     _ptr(dyt_q[1]), _ptr(xt_q[0]), _ptr(xt_q[1]), _ptr(offsets), E, m_total, n, k,
                                     _ptr(dx), dx_dtype, _ptr(dw), dw_dtype, flags, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return dx, dw


def bsq_debug_status(workspace, stream=None):
    v = I32(0)
    _check("bsq_debug_status", _lib.bsq_debug_status(_ptr(workspace), _stream(stream), ctypes.byref(v)))
    return int(v.value)


def bsq_debug_encode_e2m1(x, out=None, stream=None):
    _dev(x, "x", (torch.float32,))
    out = _empty(stream, x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    _check("bsq_debug_encode_e2m1", _lib.bsq_debug_encode_e2m1(_ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out


def bsq_debug_encode_e4m3(x, out=None, stream=None):
    _dev(x, "x", (torch.float32,))
    out = _empty(stream, x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    _check("bsq_debug_encode_e4m3", _lib.bsq_debug_encode_e4m3(_ptr(x), _ptr(out), x.numel(), _stream(stream)))
    return out
