"""Pins for the oracle's NVFP4-variant and MXFP8 quantizers.

Hand-worked fixtures, invariants the pages motivate (per-token scaling is
batch invariant and leaks nothing across tokens: "Composer 2 Technical Report"
section 6.1 and "Cursor Composer 2 report deep dive" section 1), exact
power-of-two and sign symmetries, block-permutation equivariance, round-trip
error bounds, and cross-checks against torch's float8 cast.
"""
import math

import numpy as np
import pytest
import torch

from conftest import bf16, golden_lines
from workloads import bf16_bits_to_f32, make_quantize_input, normal_bf16

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _unpack(codes):
    lo, hi = codes & 15, codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def _golden_row():
    d = {}
    for ln in golden_lines("nvfp4v_worked_row.txt"):
        k, v = ln.split(":", 1)
        d[k] = v.split()
    return d


def test_nvfp4v_worked_row(orc):
    g = _golden_row()
    x = bf16([[float(v) for v in g["x"]]])
    assert np.array_equal(bf16_bits_to_f32(x)[0], np.array([float(v) for v in g["x"]], np.float32))
    codes, bscale, rscale = orc.quantize_nvfp4v(x)
    assert rscale[0] == float(g["rscale"][0])
    assert bscale[0].tolist() == [int(b, 16) for b in g["bscale"]]
    assert _unpack(codes)[0].tolist() == [int(c, 16) for c in g["codes"]]
    assert codes[0].tolist() == [int(b, 16) for b in g["packed"]]


def test_nvfp4v_worked_row_transforms(orc):
    g = _golden_row()
    xf = np.array([[float(v) for v in g["x"]]], np.float32)
    c0, b0, r0 = orc.quantize_nvfp4v(bf16(xf))
    c1, b1, r1 = orc.quantize_nvfp4v(bf16(xf * np.float32(2.0 ** -10)))
    assert np.array_equal(c0, c1) and np.array_equal(b0, b1) and r1[0] == np.float32(2.0 ** -10)
    c2, b2, r2 = orc.quantize_nvfp4v(bf16(-xf))
    assert np.array_equal(b0, b2) and r2[0] == r0[0]
    assert np.array_equal(c2, c0 ^ 0x88)


def _pow2_value(tok):
    """'m*2^e' -> float (exact), '0' -> 0.0."""
    if "*2^" not in tok:
        return float(tok)
    m, e = tok.split("*2^")
    return math.ldexp(float(m), int(e))


def _golden_huge():
    d = {}
    for ln in golden_lines("nvfp4v_huge_row.txt"):
        k, v = ln.split(":", 1)
        d[k] = v.split()
    return d


def test_nvfp4v_huge_row(orc):
    """Block maxima above FLT_MAX / 1.75 (the branch where 448 * a_b would
    overflow): the hand-worked bytes, scale bytes 7e 7a, not 7e 7e."""
    g = _golden_huge()
    xf = np.array([[_pow2_value(t) for t in g["x"]]], np.float64)
    x = bf16(xf)
    assert np.array_equal(bf16_bits_to_f32(x).astype(np.float64), xf)  # every value bf16-exact
    codes, bscale, rscale = orc.quantize_nvfp4v(x)
    assert bscale[0].tolist() == [int(b, 16) for b in g["bscale"]]
    assert rscale.view(np.uint32)[0] == int(g["rscale_bits"][0], 16)
    assert _unpack(codes)[0].tolist() == [int(c, 16) for c in g["codes"]]
    assert codes[0].tolist() == [int(b, 16) for b in g["packed"]]
    # the same row times 2^-100 takes the unscaled branch and gives the same bytes
    c1, b1, r1 = orc.quantize_nvfp4v(bf16(xf * 2.0 ** -100))
    assert np.array_equal(c1, codes) and np.array_equal(b1, bscale)
    assert r1.view(np.uint32)[0] == int(g["rscale_bits_scaled"][0], 16)


def test_nvfp4v_power_of_two_equivariance_to_top_of_range(orc):
    """Each row scaled by the power of two that puts its max in [2^127, 2^128)
    (most rows then hold a block maximum above FLT_MAX / 1.75): the bytes of
    every row are unchanged and s_row scales exactly, whichever side of the
    2^119 switch its block maxima fall on."""
    rng = np.random.default_rng(17)
    xf = bf16_bits_to_f32(make_quantize_input(rng, 48, 256)).astype(np.float64)
    xf[5, 16:] *= 2.0 ** -12          # rows whose block maxima straddle 2^119 after scaling
    xf[6, ::16] *= 0.7
    p = 127 - np.floor(np.log2(np.abs(xf).max(axis=1)))
    big = xf * np.exp2(p)[:, None]
    assert np.all(np.abs(big).max(axis=1) >= 2.0 ** 127) and np.all(np.isfinite(big))
    assert np.mean(np.abs(big).max(axis=1) > np.finfo(np.float32).max / 1.75) > 0.3
    c0, b0, r0 = orc.quantize_nvfp4v(bf16(xf))
    c1, b1, r1 = orc.quantize_nvfp4v(bf16(big))
    assert np.array_equal(c0, c1) and np.array_equal(b0, b1)
    assert np.array_equal(r1.astype(np.float64), r0.astype(np.float64) * np.exp2(p))


def test_nvfp4v_zero_row_and_zero_block(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 16:32] = np.linspace(-3, 3, 16)
    codes, bscale, rscale = orc.quantize_nvfp4v(bf16(x))
    assert rscale[0] == 0 and not codes[0].any() and not bscale[0].any()
    assert bscale[1].tolist()[0] == 0 and bscale[1, 1] == 0x7E
    assert not codes[1, :8].any() and not codes[1, 16:].any()


def test_nvfp4v_tiny_block_scale_underflows_to_zero(orc):
    """A block whose max is below 2^-10 * A / 448 gets scale byte 0 and all-zero codes."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16] = 2.0 ** -20
    x[0, 17] = -2.0 ** -21
    codes, bscale, _ = orc.quantize_nvfp4v(bf16(x))
    assert bscale[0, 1] == 0 and not codes[0, 8:].any()


def test_nvfp4v_amax_block_and_element(orc):
    rng = np.random.default_rng(5)
    x = normal_bf16(rng, (64, 256))
    codes, bscale, rscale = orc.quantize_nvfp4v(x)
    xf = np.abs(bf16_bits_to_f32(x))
    u = _unpack(codes)
    for r in range(64):
        k = int(np.argmax(xf[r]))
        assert bscale[r, k // 16] == 0x7E
        assert (u[r, k] & 7) == 7
        assert rscale[r] == np.float32(np.float32(xf[r].max()) / np.float32(2688))


def test_nvfp4v_batch_invariance_and_prefix_independence(orc):
    rng = np.random.default_rng(6)
    x = make_quantize_input(rng, 96, 512)
    ref = orc.quantize_nvfp4v(x)
    for trial in range(6):
        perm = rng.permutation(96)
        n = int(rng.integers(1, 96))
        sub = perm[:n]
        got = orc.quantize_nvfp4v(x[sub])
        for a, b in zip(got, ref):
            assert np.array_equal(a, b[sub])
    # prefix independence: later tokens (rows) change nothing in earlier ones
    y = x.copy()
    y[50:] = make_quantize_input(rng, 46, 512, outlier_mult=1e4)
    got = orc.quantize_nvfp4v(y)
    for a, b in zip(got, ref):
        assert np.array_equal(a[:50], b[:50])


@pytest.mark.parametrize("p", [-20, -3, 1, 7, 40])
def test_nvfp4v_power_of_two_equivariance(orc, p):
    rng = np.random.default_rng(7)
    xf = bf16_bits_to_f32(normal_bf16(rng, (32, 128)))
    c0, b0, r0 = orc.quantize_nvfp4v(bf16(xf))
    c1, b1, r1 = orc.quantize_nvfp4v(bf16(xf * np.float32(2.0 ** p)))
    assert np.array_equal(c0, c1) and np.array_equal(b0, b1)
    assert np.array_equal(r1, r0 * np.float32(2.0 ** p))


def test_nvfp4v_sign_symmetry(orc):
    rng = np.random.default_rng(8)
    x = normal_bf16(rng, (32, 256))
    c0, b0, r0 = orc.quantize_nvfp4v(x)
    c1, b1, r1 = orc.quantize_nvfp4v(x ^ np.uint16(0x8000))
    assert np.array_equal(b0, b1) and np.array_equal(r0, r1)
    assert np.array_equal(c1, c0 ^ 0x88)


def test_nvfp4v_block_permutation_equivariance(orc):
    rng = np.random.default_rng(9)
    x = normal_bf16(rng, (16, 256))
    perm = rng.permutation(16)
    xp = x.reshape(16, 16, 16)[:, perm].reshape(16, 256)
    c0, b0, r0 = orc.quantize_nvfp4v(x)
    c1, b1, r1 = orc.quantize_nvfp4v(xp)
    assert np.array_equal(r0, r1)
    assert np.array_equal(b1, b0[:, perm])
    assert np.array_equal(c1, c0.reshape(16, 16, 8)[:, perm].reshape(16, 128))


def test_nvfp4v_roundtrip_bound(orc):
    rng = np.random.default_rng(10)
    x = make_quantize_input(rng, 128, 1024)
    codes, bscale, rscale = orc.quantize_nvfp4v(x)
    xhat = orc.dequant_nvfp4v(codes, bscale, rscale)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    d_exact = np.repeat(np.array([orc.e4m3_value(int(b)) for b in range(256)])[bscale]
                        * rscale[:, None].astype(np.float64), 16, axis=1)
    d = d_exact.astype(np.float32).astype(np.float64)  # the fp32 divisor d_b
    v = np.abs(xf) / d
    sat = v > 6
    half_gap = np.where(v <= 2, 0.25, np.where(v <= 4, 0.5, 1.0))
    err = np.abs(xf - xhat)
    tol = half_gap * d * (1 + 2.0 ** -20)
    assert np.all(err[~sat] <= tol[~sat])
    # saturated elements decode to exactly 6 * S_b * s_row
    assert np.allclose(err[sat], np.abs(np.abs(xf[sat]) - 6 * d_exact[sat]), rtol=0, atol=1e-12 * np.abs(xf[sat]).max())
    # normwise: 4.5-bit format, error well under 10% of the row norm
    rel = np.linalg.norm(xf - xhat, axis=1) / np.linalg.norm(xf, axis=1)
    assert rel.max() < 0.1


def _golden_blocks():
    out = []
    for ln in golden_lines("mxfp8_worked_blocks.txt"):
        lhs, rhs = ln.split("->")
        vals = dict(t.split(":") for t in lhs.replace("block:", "").split())
        sbyte, codes = rhs.split(";")
        out.append(({int(k): float(v) for k, v in vals.items()}, int(sbyte, 16),
                    {int(k): int(v, 16) for k, v in (t.split(":") for t in codes.split())}))
    return out


def test_mxfp8_worked_blocks(orc):
    for vals, sbyte, codes in _golden_blocks():
        x = np.zeros((1, 32), np.float32)
        for k, v in vals.items():
            x[0, k] = v
        c, s = orc.quantize_mxfp8_rowwise(bf16(x))
        assert s.shape == (1, 1) and s[0, 0] == sbyte, vals
        for k, v in codes.items():
            assert c[0, k] == v, (vals, k)


def test_mxfp8_rowwise_vs_frexp_and_torch(orc):
    """Shared exponent from math.frexp, element codes from torch's float8 cast."""
    rng = np.random.default_rng(11)
    x = make_quantize_input(rng, 64, 512)
    x[3] = 0
    x[4, :32] = bf16(np.full(32, 2.0 ** -130))  # subnormal bf16 block -> clamp at -127
    codes, scale = orc.quantize_mxfp8_rowwise(x)
    xf = bf16_bits_to_f32(x).astype(np.float64).reshape(64, 16, 32)
    for r in range(64):
        for b in range(16):
            blk = xf[r, b]
            A = np.abs(blk).max()
            if A == 0:
                assert scale[b, r] == 0 and not codes[r, 32 * b:32 * b + 32].any()
                continue
            sh = min(max(math.frexp(A)[1] - 1 - 8, -127), 127)
            assert scale[b, r] == sh + 127
            scaled = np.clip(blk * 2.0 ** -sh, -448, 448).astype(np.float32)
            ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, 32 * b:32 * b + 32], ref), (r, b)


def test_mxfp8_symmetries_and_bound(orc):
    rng = np.random.default_rng(12)
    x = make_quantize_input(rng, 64, 256)
    c0, s0 = orc.quantize_mxfp8_rowwise(x)
    c1, s1 = orc.quantize_mxfp8_rowwise(x ^ np.uint16(0x8000))
    assert np.array_equal(s0, s1) and np.array_equal(c1, c0 ^ 0x80)
    xf = bf16_bits_to_f32(x)
    c2, s2 = orc.quantize_mxfp8_rowwise(bf16(xf * np.float32(2.0 ** 9)))
    assert np.array_equal(c2, c0) and np.array_equal(s2.astype(int), s0.astype(int) + 9)
    xhat = orc.dequant_mxfp8(c0, s0)
    sh = np.repeat(s0.T.astype(np.float64) - 127, 32, axis=1)
    a = np.abs(xf.astype(np.float64))
    bound = np.maximum.reduce([2.0 ** -4 * a, 2.0 ** (sh - 10), a - 448 * 2.0 ** sh])
    assert np.all(np.abs(a * np.sign(xf) - xhat) <= bound)


def _segments(rng, rows, G, empty=()):
    cuts = np.sort(rng.integers(0, rows + 1, G - 1))
    off = np.concatenate([[0], cuts, [rows]]).astype(np.int32)
    for g in empty:
        off[g + 1:] = np.maximum(off[g + 1:], off[g])
        off[g + 1] = off[g]
    off[-1] = rows
    return np.maximum.accumulate(off).astype(np.int32)


def test_mxfp8_colwise_t_matches_rowwise_on_transposed_segments(orc):
    rng = np.random.default_rng(13)
    rows, cols, G = 301, 96, 6
    off = _segments(rng, rows, G)
    off[2] = off[1]  # one empty segment
    off = np.maximum.accumulate(off)
    x = make_quantize_input(rng, rows, cols)
    codes, scale = orc.quantize_mxfp8_colwise_t(x, off)
    P = 128 * (G + (rows + 127) // 128)
    assert codes.shape == (cols, P) and scale.shape == (P // 32, cols)
    covered = np.zeros(P, bool)
    for g in range(G):
        m0, m1 = int(off[g]), int(off[g + 1])
        c0 = 128 * (g + m0 // 128)
        L = 32 * ((m1 - m0 + 31) // 32)
        assert c0 % 128 == 0 and not covered[c0:c0 + L].any()
        covered[c0:c0 + L] = True
        seg = np.zeros((cols, L), np.uint16)
        seg[:, :m1 - m0] = x[m0:m1].T
        rc, rs = orc.quantize_mxfp8_rowwise(seg)
        assert np.array_equal(codes[:, c0:c0 + L], rc)
        assert np.array_equal(scale[c0 // 32:(c0 + L) // 32, :], rs)
    assert not codes[:, ~covered].any()
    assert not scale[~covered[::32], :].any()
    assert covered.sum() <= P


def test_decision_margins_flag_exactly_the_boundaries(orc):
    """Elements placed exactly on E2M1 rounding midpoints (ties) are at risk
    for any delta > 0; elements on E2M1 grid values are not (their nearest
    boundary is at least 1/12 away relative); block scales on an exact E4M3
    tie are at risk."""
    from conftest import bf16
    # one row with A = 2688, so s_row = 1.  Block 0: t = 448, d = 448, its
    # elements sit at 6 and far below 0.25 (no boundary near).  Block 1: amax
    # 6 gives t = 1, d = 1: elements on the ties 2.5, -0.75, 1.25 and on the
    # grid value 6.  Block 2: t = 448 * 1088 / 2688 = 181.33 (E4M3 neighbours
    # 176 and 192, midpoint 184: no tie).  Block 3: t = 448 * 102 / 2688 = 17,
    # the E4M3 tie between 16 and 18.
    row = np.zeros(64)
    row[:8] = [2688, 6, 4, 3, 2, 1.5, 1, 0.5]
    row[16:20] = [2.5, -0.75, 1.25, 6]
    row[32] = 1088
    row[48] = 102
    blocks, elems = orc.nvfp4v_decision_margins(bf16(row)[None, :], 2.0 ** -20)
    assert not elems[0, :8].any()
    assert elems[0, 16] and elems[0, 17] and elems[0, 18] and not elems[0, 19]
    assert not blocks[0, 0] and not blocks[0, 2] and blocks[0, 3]
    # a value far from every boundary stays safe for a large delta as well
    _, e2 = orc.nvfp4v_decision_margins(bf16(row)[None, :], 2.0 ** -6)
    assert not e2[0, :8].any()


def test_mxfp8_gather_is_rowwise_of_gathered_rows(orc):
    """The gather quantizer equals the row-wise quantizer on the identity
    index; permuting the index permutes output rows and scale columns; a
    repeated index repeats the row; out-of-range indices give zero rows."""
    from workloads import make_quantize_input
    rng = np.random.default_rng(31)
    x = make_quantize_input(rng, 40, 96)
    ident = orc.quantize_mxfp8_gather(x, np.arange(40))
    plain = orc.quantize_mxfp8_rowwise(x)
    assert np.array_equal(ident[0], plain[0]) and np.array_equal(ident[1], plain[1])
    perm = rng.permutation(40)
    pc, ps = orc.quantize_mxfp8_gather(x, perm)
    assert np.array_equal(pc, plain[0][perm]) and np.array_equal(ps, plain[1][:, perm])
    idx = np.array([3, 3, -1, 40, 7])
    gc, gs = orc.quantize_mxfp8_gather(x, idx)
    assert np.array_equal(gc[0], gc[1]) and np.array_equal(gc[0], plain[0][3])
    assert not gc[2].any() and not gc[3].any() and not gs[:, 2].any() and not gs[:, 3].any()
    assert np.array_equal(gc[4], plain[0][7])
