"""Pins for the oracle's grouped GEMMs (float64 over dequantized operands).

* Exact closed form: every NVFP4-variant element q*S_b is an integer multiple
  of 2^-10 below 2^12, so sum_k (q_a S_a)(q_w S_w) is an exact int64 sum; the
  oracle must match it after the two fp32 row scales.  MXFP8 elements are
  multiples of 2^-9 times a power of two per 32-block, so each block's partial
  sum is exact in int64.
* One-hot weights select dequantized activation columns exactly.
* Brute force with exact rationals on a tiny case.
* Segment handling: empty experts, rows attributed by offsets.
"""
from fractions import Fraction

import numpy as np
import torch

from workloads import bf16_bits_to_f32, make_quantize_input, normal_bf16, offsets_from_counts

E2M1_X2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
E4M3_X512 = None


def e4m3_x512():
    global E4M3_X512
    if E4M3_X512 is None:
        v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        v = np.where(np.isnan(v), 0, v) * 512
        assert np.all(v == np.round(v))
        E4M3_X512 = v.astype(np.int64)
    return E4M3_X512


def nvfp4v_int(codes, bscale):
    """Elements as integers in units of 2^-10 (before the row scale)."""
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1)
    return E2M1_X2[nib] * np.repeat(e4m3_x512()[bscale], 16, axis=1)


def _quantized_moe(orc, rng, counts, n, k):
    off = offsets_from_counts(counts)
    M = int(off[-1])
    a = orc.quantize_nvfp4v(make_quantize_input(rng, M, k))
    w = orc.quantize_nvfp4v(normal_bf16(rng, (len(counts) * n, k), 0.02))
    return off, a, w


def test_fwd_matches_exact_int64(orc):
    rng = np.random.default_rng(21)
    counts = [37, 0, 70, 1, 20]
    n, k = 48, 512
    off, a, w = _quantized_moe(orc, rng, counts, n, k)
    y = orc.grouped_gemm_fwd(a, w, off)
    ai = nvfp4v_int(a[0], a[1])
    wi = nvfp4v_int(w[0], w[1])
    for e in range(len(counts)):
        m0, m1 = off[e], off[e + 1]
        if m1 == m0:
            continue
        exact = ai[m0:m1] @ wi[e * n:(e + 1) * n].T          # int64, exact
        absum = np.abs(ai[m0:m1]) @ np.abs(wi[e * n:(e + 1) * n]).T
        scale = a[2][m0:m1, None].astype(np.float64) * w[2][None, e * n:(e + 1) * n].astype(np.float64)
        ref = exact.astype(np.float64) * 2.0 ** -20 * scale
        bound = absum.astype(np.float64) * 2.0 ** -20 * np.abs(scale) * 1e-12
        assert np.all(np.abs(y[m0:m1] - ref) <= bound + 1e-300)
    assert y.shape == (off[-1], n)


def test_fwd_full_depth_rows_exact(orc):
    rng = np.random.default_rng(22)
    counts = [5, 3]
    n, k = 16, 7168
    off, a, w = _quantized_moe(orc, rng, counts, n, k)
    rows = np.array([0, 4, 5, 7])
    y = orc.grouped_gemm_fwd(a, w, off, rows=rows)
    ai = nvfp4v_int(a[0][rows], a[1][rows])
    wi = nvfp4v_int(w[0], w[1])
    for i, r in enumerate(rows):
        e = 0 if r < 5 else 1
        exact = ai[i] @ wi[e * n:(e + 1) * n].T
        ref = exact.astype(np.float64) * 2.0 ** -20 * float(a[2][r]) * w[2][e * n:(e + 1) * n].astype(np.float64)
        assert np.allclose(y[i], ref, rtol=1e-12, atol=0)


def test_fwd_one_hot_weights_select_columns(orc):
    rng = np.random.default_rng(23)
    M, K, N, E = 40, 128, 24, 2
    a = orc.quantize_nvfp4v(make_quantize_input(rng, M, K))
    cols = rng.integers(0, K, size=(E, N))
    codes = np.zeros((E * N, K // 2), np.uint8)
    bsc = np.zeros((E * N, K // 16), np.uint8)
    for e in range(E):
        for j in range(N):
            c = cols[e, j]
            codes[e * N + j, c // 2] = 2 << (4 * (c % 2))   # E2M1 code 2 = 1.0
            bsc[e * N + j, c // 16] = 0x38                   # E4M3 1.0
    rs = np.ones(E * N, np.float32)
    off = np.array([0, 15, M], np.int32)
    y = orc.grouped_gemm_fwd(a, (codes, bsc, rs), off)
    ahat = orc.dequant_nvfp4v(*a)
    for e in range(E):
        assert np.array_equal(y[off[e]:off[e + 1]], ahat[off[e]:off[e + 1]][:, cols[e]])


def test_fwd_bruteforce_rationals(orc):
    rng = np.random.default_rng(24)
    M, N, K = 3, 2, 32
    a = orc.quantize_nvfp4v(make_quantize_input(rng, M, K))
    w = orc.quantize_nvfp4v(normal_bf16(rng, (N, K)))
    y = orc.grouped_gemm_fwd(a, w, np.array([0, M], np.int32))
    e2m1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]

    def val(q, r, k):
        byte = int(q[0][r, k // 2])
        c = byte & 15 if k % 2 == 0 else byte >> 4
        mag = e2m1[c & 7] * Fraction(float(torch.tensor([int(q[1][r, k // 16])], dtype=torch.uint8)
                                           .view(torch.float8_e4m3fn).float())) * Fraction(float(q[2][r]))
        return -mag if c & 8 else mag

    for m in range(M):
        for n in range(N):
            s = sum(val(a, m, k) * val(w, n, k) for k in range(K))
            assert abs(Fraction(y[m, n]) - s) <= abs(s) * Fraction(1, 10 ** 13)


def _mx_exact_tn(ac, asc, bc, bsc):
    """sum over the contiguous axis of two MXFP8 matrices, block partial sums
    exact in int64, combined with their power-of-two factors in float64."""
    t = e4m3_x512()
    A = t[ac].reshape(ac.shape[0], -1, 32)
    B = t[bc].reshape(bc.shape[0], -1, 32)
    part = np.einsum("ibk,jbk->ijb", A, B)  # int64, exact per block
    asc, bsc = asc.T, bsc.T  # block-major scales -> [rows, blocks]
    sh = (asc.astype(np.int64) - 127)[:, None, :] + (bsc.astype(np.int64) - 127)[None, :, :]
    return (part.astype(np.float64) * np.exp2(sh - 18)).sum(-1), (np.abs(part).astype(np.float64) *
                                                                np.exp2(sh - 18)).sum(-1)


def test_dgrad_matches_exact_blocks(orc):
    rng = np.random.default_rng(25)
    counts = [20, 0, 33, 7]
    E, n, k = len(counts), 96, 64
    off = offsets_from_counts(counts)
    M = int(off[-1])
    dy = normal_bf16(rng, (M, n), 1e-3)
    w = normal_bf16(rng, (E * n, k), 0.02)
    dy_q = orc.quantize_mxfp8_rowwise(dy)
    wt_q = orc.quantize_mxfp8_colwise_t(w, np.arange(E + 1, dtype=np.int32) * n)
    dx = orc.grouped_gemm_dgrad(dy_q, wt_q, off, n)
    woff = np.arange(E + 1) * n
    for e in range(E):
        m0, m1 = off[e], off[e + 1]
        if m0 == m1:
            continue
        c0 = 128 * (e + woff[e] // 128)
        ref, absum = _mx_exact_tn(dy_q[0][m0:m1], dy_q[1][:, m0:m1], wt_q[0][:, c0:c0 + n],
                                  wt_q[1][c0 // 32:(c0 + n) // 32, :])
        assert np.all(np.abs(dx[m0:m1] - ref) <= 1e-12 * absum + 1e-300)


def test_wgrad_matches_exact_blocks_and_outer_products(orc):
    rng = np.random.default_rng(26)
    counts = [45, 0, 3, 64]
    E, n, k = len(counts), 64, 96
    off = offsets_from_counts(counts)
    M = int(off[-1])
    dy = normal_bf16(rng, (M, n), 1e-3)
    x = make_quantize_input(rng, M, k)
    dyt = orc.quantize_mxfp8_colwise_t(dy, off)
    xt = orc.quantize_mxfp8_colwise_t(x, off)
    dw = orc.grouped_gemm_wgrad(dyt, xt, off)
    for e in range(E):
        m0, m1 = int(off[e]), int(off[e + 1])
        if m0 == m1:
            assert not dw[e].any()
            continue
        c0 = 128 * (e + m0 // 128)
        L = 32 * ((m1 - m0 + 31) // 32)
        ref, absum = _mx_exact_tn(dyt[0][:, c0:c0 + L], dyt[1][c0 // 32:(c0 + L) // 32, :],
                                  xt[0][:, c0:c0 + L], xt[1][c0 // 32:(c0 + L) // 32, :])
        assert np.all(np.abs(dw[e] - ref) <= 1e-12 * absum + 1e-300)
        # independent structure: sum of per-token outer products of the
        # dequantized token vectors
        dyh = orc.dequant_mxfp8(dyt[0][:, c0:c0 + L], dyt[1][c0 // 32:(c0 + L) // 32, :])
        xh = orc.dequant_mxfp8(xt[0][:, c0:c0 + L], xt[1][c0 // 32:(c0 + L) // 32, :])
        acc = np.zeros((n, k))
        for j in range(m1 - m0):
            acc += np.outer(dyh[:, j], xh[:, j])
        assert np.allclose(dw[e], acc, rtol=1e-12, atol=1e-300)
        assert not dyh[:, m1 - m0:].any() and not xh[:, m1 - m0:].any()


def test_fwd_mxfp8_matches_exact_blocks(orc):
    """All-MXFP8 forward: per-expert products equal the exact int64 block sums
    (ROWWISE codes of X rows against ROWWISE codes of the expert's weight
    rows); rows of empty experts do not exist and every row is attributed to
    the expert its offsets give."""
    rng = np.random.default_rng(28)
    counts = [9, 0, 40, 1]
    E, n, k = len(counts), 64, 96
    off = offsets_from_counts(counts)
    M = int(off[-1])
    x = make_quantize_input(rng, M, k)
    w = normal_bf16(rng, (E * n, k), 0.02)
    x_q, w_q = orc.quantize_mxfp8_rowwise(x), orc.quantize_mxfp8_rowwise(w)
    y = orc.grouped_gemm_fwd_mxfp8(x_q, w_q, off)
    ya = orc.grouped_gemm_fwd_mxfp8(x_q, w_q, off, absolute=True)
    for e in range(E):
        m0, m1 = int(off[e]), int(off[e + 1])
        if m0 == m1:
            continue
        ref, absum = _mx_exact_tn(x_q[0][m0:m1], x_q[1][:, m0:m1], w_q[0][e * n:(e + 1) * n],
                                  w_q[1][:, e * n:(e + 1) * n])
        assert np.all(np.abs(y[m0:m1] - ref) <= 1e-12 * absum + 1e-300)
        # absolute sums: the same exact block sums over magnitudes (sign bit 7 cleared)
        ref_abs, _ = _mx_exact_tn(x_q[0][m0:m1] & 0x7F, x_q[1][:, m0:m1], w_q[0][e * n:(e + 1) * n] & 0x7F,
                                  w_q[1][:, e * n:(e + 1) * n])
        assert np.allclose(ya[m0:m1], ref_abs, rtol=1e-12, atol=0)
    rows = np.array([M - 1, 0, 20])
    assert np.array_equal(orc.grouped_gemm_fwd_mxfp8(x_q, w_q, off, rows=rows), y[rows])


def test_bf16_gemm_exact_on_integers_and_rationals(orc):
    """bf16 baseline: small-integer operands give exact int64 sums; a tiny
    case against exact rationals; rows follow their expert's weights."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(29)
    counts = [5, 0, 12, 3]
    E, n, k = len(counts), 8, 96
    off = offsets_from_counts(counts)
    M = int(off[-1])
    xi = rng.integers(-16, 17, (M, k))
    wi = rng.integers(-16, 17, (E * n, k))
    y = orc.grouped_gemm_bf16(f32_to_bf16_bits(xi.astype(np.float32)), f32_to_bf16_bits(wi.astype(np.float32)), off)
    for e in range(E):
        m0, m1 = int(off[e]), int(off[e + 1])
        assert np.array_equal(y[m0:m1], (xi[m0:m1] @ wi[e * n:(e + 1) * n].T).astype(np.float64))
    xb = normal_bf16(rng, (3, 5))
    wb = normal_bf16(rng, (2, 5))
    yb = orc.grouped_gemm_bf16(xb, wb, np.array([0, 3], np.int32))
    xv, wv = bf16_bits_to_f32(xb), bf16_bits_to_f32(wb)
    for m in range(3):
        for j in range(2):
            exact = sum(Fraction(float(xv[m, q])) * Fraction(float(wv[j, q])) for q in range(5))
            assert abs(Fraction(yb[m, j]) - exact) <= abs(exact) * Fraction(1, 10 ** 14)


def test_single_expert_is_dense(orc):
    """With offsets [0, M] the grouped fwd equals one dense product of the
    dequantized matrices, and dequantized values are the bf16 inputs to
    within the format's error."""
    rng = np.random.default_rng(27)
    x = make_quantize_input(rng, 33, 64)
    w = normal_bf16(rng, (16, 64))
    a_q, w_q = orc.quantize_nvfp4v(x), orc.quantize_nvfp4v(w)
    y = orc.grouped_gemm_fwd(a_q, w_q, np.array([0, 33], np.int32))
    ai, wi = nvfp4v_int(a_q[0], a_q[1]), nvfp4v_int(w_q[0], w_q[1])
    ref = (ai @ wi.T).astype(np.float64) * 2.0 ** -20 * np.outer(a_q[2].astype(np.float64), w_q[2].astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-12, atol=0)
    yf = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    assert np.linalg.norm(y - yf) / np.linalg.norm(yf) < 0.2


def packed_exact_weights(rng, rows, k, jlo=-6, jhi=6):
    """bf16 weight rows the NVFP4 variant represents exactly: block 0 of each
    row holds a 6 * 448 = 2688 element (so A = 2688 and s_row = A / 2688 = 1)
    and E2M1 multiples of 448 (S_0 = E4M3(448 * 2688 / 2688) = 448); every
    other 16-block holds a +-6 * 2^j element and E2M1 multiples of 2^j
    (S_b = E4M3(448 * 6 * 2^j / 2688) = 2^j).  Returns (bf16 bits, float64)."""
    from workloads import f32_to_bf16_bits
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    nb = k // 16
    s = np.ones((rows, nb)) * 448.0
    s[:, 1:] = 2.0 ** rng.integers(jlo, jhi + 1, (rows, nb - 1))
    v = mags[rng.integers(0, 8, (rows, k))] * np.where(rng.random((rows, k)) < 0.5, -1, 1)
    v[:, ::16] = 6 * np.where(rng.random((rows, nb)) < 0.5, -1, 1)  # every block reaches its max
    w = v * np.repeat(s, 16, axis=1)
    bits = f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), w)
    return bits, w


def test_w4a16_exact_on_representable_weights(orc):
    """Frozen-expert GEMM: weights the packed format holds exactly decode to
    themselves, and with integer activations the grouped product equals the
    plain float64 product of the original bf16 inputs, expert by expert
    (empty expert, one-row expert, row order given by offsets)."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(31)
    counts = [7, 0, 1, 20]
    E, n, k = len(counts), 12, 64
    off = offsets_from_counts(counts)
    M = int(off[-1])
    wb, wv = packed_exact_weights(rng, E * n, k)
    w_q = orc.quantize_nvfp4v(wb)
    assert np.all(w_q[2] == 1.0)
    assert np.array_equal(orc.dequant_nvfp4v(*w_q), wv)
    xi = rng.integers(-8, 9, (M, k)).astype(np.float64)
    y = orc.grouped_gemm_w4a16(f32_to_bf16_bits(xi.astype(np.float32)), w_q, off)
    for e in range(E):
        m0, m1 = int(off[e]), int(off[e + 1])
        assert np.array_equal(y[m0:m1], xi[m0:m1] @ wv[e * n:(e + 1) * n].T)
    sub = np.array([M - 1, 0, 8])
    assert np.array_equal(orc.grouped_gemm_w4a16(f32_to_bf16_bits(xi.astype(np.float32)), w_q, off, rows=sub),
                          y[sub])


def test_w4a16_applies_row_scale_and_block_scales(orc):
    """Against exact rationals on a tiny case with arbitrary (non power of
    two) row and block scales: Y = sum_k x * e2m1 * S_b, times s_row."""
    rng = np.random.default_rng(32)
    x = normal_bf16(rng, (3, 32))
    w = normal_bf16(rng, (4, 32), 0.02)
    w_q = orc.quantize_nvfp4v(w)
    y = orc.grouped_gemm_w4a16(x, w_q, np.array([0, 3], np.int32))
    xv = bf16_bits_to_f32(x)
    wi = nvfp4v_int(w_q[0], w_q[1])
    for m in range(3):
        for j in range(4):
            exact = sum(Fraction(float(xv[m, q])) * Fraction(int(wi[j, q]), 1024) for q in range(32))
            exact *= Fraction(float(w_q[2][j]))
            assert abs(Fraction(y[m, j]) - exact) <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)
