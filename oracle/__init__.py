"""CPU oracle for the block-scaled MoE expert GEMM path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package.  It shares no code with
the HIP library (``block_scaled_precision_bsq_amd``) and never imports it.

Bit-level codecs and quantizers live in ``bsq_oracle.c`` (plain C, IEEE binary32
arithmetic, no FMA contraction); this module wraps them with numpy and adds the
grouped GEMMs, which are written as "dequantize to float64, then multiply"
(``numpy.matmul`` on float64 serves as the matmul step).

Sources: "Composer 2 Technical Report" (papercache.org summary), section 6.1
(NVFP4 variant in the MoE forward: E2M1 values, E4M3 scale per 16-element
block, FP32 scale per token; standard MXFP8 in the backward: E4M3 values,
E8M0 scale per 32; IEEE division for NVFP4 quantization) and "Cursor Composer 2
report deep dive" (machinelearningatscale), section 1 "The kernel section".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (``force`` recompiles even if present)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        U8 = ctypes.c_uint8
        L.orc_e2m1_value.argtypes = [U8]; L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [U8]; L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [U8]; L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]; L.orc_e2m1_encode.restype = U8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]; L.orc_e4m3_encode.restype = U8
        L.orc_e2m1_encode_array.argtypes = [P, P, I64]; L.orc_e2m1_encode_array.restype = None
        L.orc_e4m3_encode_array.argtypes = [P, P, I64]; L.orc_e4m3_encode_array.restype = None
        L.orc_quantize_nvfp4v.argtypes = [P, I64, I64, I64, P, P, P]; L.orc_quantize_nvfp4v.restype = None
        L.orc_dequant_nvfp4v.argtypes = [P, P, P, I64, I64, P]; L.orc_dequant_nvfp4v.restype = None
        L.orc_quantize_mxfp8_rowwise.argtypes = [P, I64, I64, I64, P, P]
        L.orc_quantize_mxfp8_rowwise.restype = None
        L.orc_colwise_padded_cols.argtypes = [I32, I64]; L.orc_colwise_padded_cols.restype = I64
        L.orc_quantize_mxfp8_colwise_t.argtypes = [P, I64, I64, I64, P, I32, P, P]
        L.orc_quantize_mxfp8_colwise_t.restype = None
        L.orc_dequant_mxfp8.argtypes = [P, P, I64, I64, I64, I64, I64, P]; L.orc_dequant_mxfp8.restype = None
        L.orc_set_num_threads.argtypes = [ctypes.c_int]; L.orc_set_num_threads.restype = None
        L.orc_max_threads.argtypes = []; L.orc_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16)")
    return x


def set_num_threads(n: int) -> None:
    """Threads of the C oracle's parallel loops (timing only; results do not
    depend on it)."""
    lib().orc_set_num_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ------------------------------------------------------------------ codecs

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(b)


def e8m0_value(b: int) -> float:
    return lib().orc_e8m0_value(b)


def e2m1_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e2m1_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


E2M1_TABLE = None
E4M3_TABLE = None
E8M0_TABLE = None


def tables():
    """Decode tables (float64) for all 16 E2M1, 256 E4M3 and 256 E8M0 codes."""
    global E2M1_TABLE, E4M3_TABLE, E8M0_TABLE
    if E2M1_TABLE is None:
        E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)])
        E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)])
        E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)])
    return E2M1_TABLE, E4M3_TABLE, E8M0_TABLE


# -------------------------------------------------------------- quantizers

def quantize_nvfp4v(x_bf16: np.ndarray):
    """NVFP4 variant of each row of a [rows, cols] bf16 matrix.

    Returns (codes [rows, cols/2] u8, bscale [rows, cols/16] u8 (E4M3),
    rscale [rows] f32 (decode scale)).
    """
    x = _bf16(x_bf16)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    codes = np.empty((rows, cols // 2), np.uint8)
    bscale = np.empty((rows, cols // 16), np.uint8)
    rscale = np.empty((rows,), np.float32)
    lib().orc_quantize_nvfp4v(_ptr(x), rows, cols, cols, _ptr(codes), _ptr(bscale), _ptr(rscale))
    return codes, bscale, rscale


def dequant_nvfp4v(codes, bscale, rscale) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    bscale = np.ascontiguousarray(bscale, np.uint8)
    rscale = np.ascontiguousarray(rscale, np.float32)
    rows, half = codes.shape
    out = np.empty((rows, 2 * half), np.float64)
    lib().orc_dequant_nvfp4v(_ptr(codes), _ptr(bscale), _ptr(rscale), rows, 2 * half, _ptr(out))
    return out


def quantize_mxfp8_rowwise(x_bf16: np.ndarray):
    """MXFP8 with blocks of 32 along each row.  Returns (codes [rows, cols],
    scale [cols/32, rows]) -- scales block-major."""
    x = _bf16(x_bf16)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    codes = np.empty((rows, cols), np.uint8)
    scale = np.empty((cols // 32, rows), np.uint8)
    lib().orc_quantize_mxfp8_rowwise(_ptr(x), rows, cols, cols, _ptr(codes), _ptr(scale))
    return codes, scale


def nvfp4v_decision_margins(x_bf16: np.ndarray, delta: float):
    """Which decisions of the NVFP4-variant quantizer a divide with relative
    error up to ``delta`` could change ("Composer 2 Technical Report", section
    6.1: the quantizer needs IEEE division; a fast approximate divide made
    training diverge).  With exact division, block b's scale byte is
    E4M3(448 a_b / A) and element x's code is E2M1(x / d_b); a perturbed
    divide can change a decision only if the exact argument lies within
    ``delta`` (relative) of a rounding boundary of its encoder, i.e. if the
    encoder maps arg * (1 - delta) and arg * (1 + delta) to different codes.
    Returns (blocks_at_risk [rows, cols/16], elements_at_risk [rows, cols]),
    the elements judged against the exact-division d_b."""
    x = _bf16(x_bf16)
    rows, cols = x.shape
    codes, bscale, rscale = quantize_nvfp4v(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a_b = np.abs(xf).reshape(rows, cols // 16, 16).max(-1)
    A = a_b.max(-1, keepdims=True) if cols else np.zeros((rows, 1))
    t = np.divide(448.0 * a_b, A, out=np.zeros_like(a_b), where=A > 0)
    blocks = e4m3_encode(t * (1 - delta)) != e4m3_encode(t * (1 + delta))
    _, e4m3_tab, _ = tables()
    d = (e4m3_tab[bscale].astype(np.float32) * rscale[:, None].astype(np.float32)).astype(np.float64)  # RN32
    d = np.repeat(d, 16, axis=1)
    q = np.divide(xf, d, out=np.zeros_like(xf), where=d > 0)
    elems = e2m1_encode(q * (1 - delta)) != e2m1_encode(q * (1 + delta))
    return blocks, elems


def quantize_mxfp8_gather(x_bf16: np.ndarray, row_index):
    """MXFP8 ROWWISE of the rows x[row_index] (the token permutation of an
    expert dispatch; "Composer 2 Technical Report" section 6.1, tokens
    quantized to MXFP8 before dispatch).  An index outside [0, rows) stands
    for an all-zero row."""
    x = _bf16(x_bf16)
    idx = np.asarray(row_index, np.int64)
    ok = (idx >= 0) & (idx < x.shape[0])
    g = np.zeros((len(idx), x.shape[1]), np.uint16)
    g[ok] = x[idx[ok]]
    return quantize_mxfp8_rowwise(g)


def padded_cols(ngroups: int, rows: int) -> int:
    return int(lib().orc_colwise_padded_cols(ngroups, rows))


def segment_start(g: int, offsets) -> int:
    """First padded column of segment g in the COLWISE_T layout."""
    return 128 * (g + int(offsets[g]) // 128)


def quantize_mxfp8_colwise_t(x_bf16: np.ndarray, offsets):
    """MXFP8 with blocks of 32 running down the rows of each segment
    ``[offsets[g], offsets[g+1])``; output transposed and per-segment padded.
    Returns (codes [cols, P], scale [P/32, cols]) -- scales block-major."""
    x = _bf16(x_bf16)
    rows, cols = x.shape
    off = np.ascontiguousarray(offsets, np.int32)
    G = len(off) - 1
    P = padded_cols(G, rows)
    codes = np.empty((cols, P), np.uint8)
    scale = np.empty((P // 32, cols), np.uint8)
    lib().orc_quantize_mxfp8_colwise_t(_ptr(x), rows, cols, cols, _ptr(off), G, _ptr(codes), _ptr(scale))
    return codes, scale


def dequant_mxfp8(codes, scale) -> np.ndarray:
    """Dequantize a matrix whose MXFP8 blocks run along its rows (a ROWWISE
    output, or a COLWISE_T output read as [cols, P]); ``scale`` is
    block-major, [cols/32, rows]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scale = np.ascontiguousarray(scale, np.uint8)
    rows, cols = codes.shape
    if scale.shape != (cols // 32, rows):
        raise ValueError("scale must be block-major [cols/32, rows]")
    out = np.empty((rows, cols), np.float64)
    lib().orc_dequant_mxfp8(_ptr(codes), _ptr(scale), rows, cols, cols, 1, rows, _ptr(out))
    return out


# ------------------------------------------------------------ grouped GEMMs

def _expert_of_rows(offsets, rows):
    off = np.asarray(offsets, np.int64)
    return np.searchsorted(off, rows, side="right") - 1


def grouped_gemm_fwd(a_q, w_q, offsets, rows=None) -> np.ndarray:
    """Forward expert GEMM over NVFP4-variant operands, in float64.

    ``a_q`` = (codes [M, K/2], bscale [M, K/16], rscale [M]) for the
    expert-sorted activations; ``w_q`` = the same for the weights stacked as
    [E*N, ...] (expert e owns rows e*N .. e*N+N-1).  Returns
    Y[m, n] = sum_k A_hat[m, k] * W_hat_e[n, k] for m in segment e, over all m
    (or only the listed ``rows``, in that order).
    """
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    M = a_q[0].shape[0]
    N = w_q[0].shape[0] // E
    rows = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    exp_of = _expert_of_rows(off, rows)
    y = np.zeros((len(rows), N), np.float64)
    for e in np.unique(exp_of):
        sel = np.nonzero(exp_of == e)[0]
        r = rows[sel]
        a_hat = dequant_nvfp4v(a_q[0][r], a_q[1][r], a_q[2][r])
        sl = slice(e * N, (e + 1) * N)
        w_hat = dequant_nvfp4v(w_q[0][sl], w_q[1][sl], w_q[2][sl])
        y[sel] = a_hat @ w_hat.T
    return y


def grouped_gemm_fwd_mxfp8(x_q, w_q, offsets, rows=None, absolute=False) -> np.ndarray:
    """All-MXFP8 forward expert GEMM ("Composer 2 Technical Report" section
    3.1, continued pretraining in MXFP8; "Scaling and Optimizing Frontier
    Model Training", MXFP8 expert kernels), in float64:
    Y[m, j] = sum_k X_hat[m, k] * W_hat_e[j, k] for m in segment e.

    ``x_q`` = ROWWISE MXFP8 of X [M, K]; ``w_q`` = ROWWISE MXFP8 of the
    weights stacked as [E*N, K] (expert e owns rows e*N .. e*N+N-1); scales
    block-major.  ``absolute=True``: sums of absolute products instead.
    """
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    M = x_q[0].shape[0]
    N = w_q[0].shape[0] // E
    rows = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    exp_of = _expert_of_rows(off, rows)
    y = np.zeros((len(rows), N), np.float64)
    for e in np.unique(exp_of):
        sel = np.nonzero(exp_of == e)[0]
        r = rows[sel]
        x_hat = dequant_mxfp8(x_q[0][r], x_q[1][:, r])
        sl = slice(int(e) * N, (int(e) + 1) * N)
        w_hat = dequant_mxfp8(w_q[0][sl], w_q[1][:, sl])
        if absolute:
            x_hat, w_hat = np.abs(x_hat), np.abs(w_hat)
        y[sel] = x_hat @ w_hat.T
    return y


def grouped_gemm_bf16(x_bf16, w_bf16, offsets, rows=None) -> np.ndarray:
    """bf16 baseline of the forward expert GEMM ("Scaling and Optimizing
    Frontier Model Training", MXFP8 expert kernels, compared with BF16), in
    float64: Y[m, j] = sum_k X[m, k] * W_e[j, k] for m in segment e, with the
    bf16 inputs taken exactly."""
    x, w = _bf16(x_bf16), _bf16(w_bf16)
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    N = w.shape[0] // E
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows, np.int64)
    exp_of = _expert_of_rows(off, rows)
    y = np.zeros((len(rows), N), np.float64)
    f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for e in np.unique(exp_of):
        sel = np.nonzero(exp_of == e)[0]
        y[sel] = f64(x[rows[sel]]) @ f64(w[int(e) * N:(int(e) + 1) * N]).T
    return y


def grouped_gemm_w4a16(x_bf16, w_q, offsets, rows=None) -> np.ndarray:
    """Frozen-expert forward GEMM over packed weights ("Scaling and Optimizing
    Frontier Model Training", low-precision expert quantization: frozen
    experts kept in a packed low-precision format and dequantized to bf16 on
    the fly), in float64: Y[m, j] = sum_k X[m, k] * W_hat_e[j, k] for m in
    segment e, with the bf16 activations taken exactly and W_hat the decoded
    NVFP4-variant weights (codes, bscale, rscale) stacked as [E*N, K]."""
    x = _bf16(x_bf16)
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    N = w_q[0].shape[0] // E
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows, np.int64)
    exp_of = _expert_of_rows(off, rows)
    y = np.zeros((len(rows), N), np.float64)
    f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for e in np.unique(exp_of):
        sel = np.nonzero(exp_of == e)[0]
        sl = slice(int(e) * N, (int(e) + 1) * N)
        y[sel] = f64(x[rows[sel]]) @ dequant_nvfp4v(w_q[0][sl], w_q[1][sl], w_q[2][sl]).T
    return y


def grouped_gemm_dgrad(dy_q, wt_q, offsets, n, rows=None, absolute=False) -> np.ndarray:
    """dX[m, k] = sum_n dY_hat[m, n] * W_hat_e[n, k] (float64).

    ``dy_q`` = ROWWISE MXFP8 of dY [M, N]; ``wt_q`` = COLWISE_T MXFP8 of the
    weights [E*N, K] with segments of N rows per expert, i.e. codes [K, P_w].
    ``absolute=True`` returns sum_n |dY_hat| |W_hat| instead (the scale of the
    rounding error of any summation of these products).
    """
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    M = dy_q[0].shape[0]
    K = wt_q[0].shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    exp_of = _expert_of_rows(off, rows)
    woff = np.arange(E + 1, dtype=np.int64) * n
    out = np.zeros((len(rows), K), np.float64)
    for e in np.unique(exp_of):
        sel = np.nonzero(exp_of == e)[0]
        r = rows[sel]
        dy_hat = dequant_mxfp8(dy_q[0][r], dy_q[1][:, r])
        c0 = segment_start(int(e), woff)
        wt_hat = dequant_mxfp8(wt_q[0][:, c0:c0 + n], wt_q[1][c0 // 32:c0 // 32 + n // 32, :])
        if absolute:
            dy_hat, wt_hat = np.abs(dy_hat), np.abs(wt_hat)
        out[sel] = dy_hat @ wt_hat.T
    return out


def grouped_gemm_wgrad(dyt_q, xt_q, offsets, experts=None, absolute=False) -> dict:
    """dW_e[n, k] = sum_{m in segment e} dY_hat[m, n] * X_hat[m, k] (float64).

    ``dyt_q`` / ``xt_q`` = COLWISE_T MXFP8 of dY [M, N] and X [M, K] with the
    expert offsets.  Returns {e: dW_e [N, K]} for the listed (default: all)
    experts; an empty expert gives zeros.  ``absolute=True``: sums of
    absolute products instead.
    """
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    experts = range(E) if experts is None else experts
    res = {}
    for e in experts:
        m_e = int(off[e + 1] - off[e])
        c0 = segment_start(int(e), off)
        L = 32 * ((m_e + 31) // 32)
        dyt = dequant_mxfp8(dyt_q[0][:, c0:c0 + L], dyt_q[1][c0 // 32:c0 // 32 + L // 32, :])
        xt = dequant_mxfp8(xt_q[0][:, c0:c0 + L], xt_q[1][c0 // 32:c0 // 32 + L // 32, :])
        if absolute:
            dyt, xt = np.abs(dyt), np.abs(xt)
        res[int(e)] = dyt @ xt.T
    return res


def swiglu(gu: np.ndarray) -> np.ndarray:
    """Harness activation between the two forward GEMMs (not on the pages):
    [gate | up] along the last axis, H = silu(gate) * up, in float64, with
    silu(g) = g / (1 + e^-g) written as g e^g / (1 + e^g) for g < 0 so that
    no exponential overflows."""
    g, u = np.split(np.asarray(gu, np.float64), 2, axis=-1)
    t = np.exp(-np.abs(g))
    return np.where(g >= 0, g, g * t) / (1.0 + t) * u


def round_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one rounding to nearest even.

    bf16 keeps 8 significant bits, exponents down to -126 (normal) and a
    subnormal quantum of 2**-133; magnitudes at or beyond the halfway point
    above the largest finite value become infinity.  NaN is not handled.
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    m, e = np.frexp(a)                      # a = m * 2**e, m in [0.5, 1)
    e = np.maximum(e, -125)                 # below 2**-126 the quantum stops shrinking
    q = np.ldexp(1.0, e - 8)                # quantum of the 8-significant-bit grid
    r = np.rint(a / q) * q                  # a / q and the product are exact in float64
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # r is a bf16 value
    return np.where(np.signbit(x), bits | np.uint16(0x8000), bits).astype(np.uint16)


def swiglu_bf16(gu_bf16: np.ndarray) -> np.ndarray:
    """H = silu(gate) * up of bf16 [gate | up] rows, computed in float64 and
    rounded once to bf16 (bit patterns)."""
    g = _bf16(gu_bf16)
    f = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return round_bf16(swiglu(f))
