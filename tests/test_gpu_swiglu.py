"""GPU parity of the fused SwiGLU + NVFP4-variant quantization through the C
ABI.  H is compared with the oracle's float64 SwiGLU rounded once to bf16: the
kernel evaluates silu in binary32, so an element may land one bf16 ulp away
when the exact value sits next to a rounding boundary.  Where the kernel's H
row equals the oracle's, codes, block scales and the row scale must equal the
oracle's quantization of that row bit for bit; in the other rows every
dequantized element must lie within its block's step d_b of the oracle's H
(plus the ulp it moved)."""
import numpy as np
import pytest
import torch

from workloads import bf16_bits_to_f32, f32_to_bf16_bits, rng_for

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def _gu(rng, rows, inter):
    """Gate/up GEMM outputs: N(0, 2) with a few large entries and exact zeros."""
    g = rng.standard_normal((rows, 2 * inter), dtype=np.float32) * np.float32(2.0)
    g[rng.random((rows, 2 * inter)) < 0.002] *= np.float32(40.0)
    g[rng.random((rows, 2 * inter)) < 0.001] = 0.0
    return f32_to_bf16_bits(g)


def _check(orc, bsq, gu_bits, h_got, q_got):
    rows = gu_bits.shape[0]
    h_ref = orc.swiglu_bf16(gu_bits)
    hg = h_got.view(np.uint16)
    diff = hg != h_ref
    # the two differ by at most one bf16 ulp (adjacent bit patterns, same sign)
    sgn = (hg >> 15) == (h_ref >> 15)
    assert np.all(~diff | (sgn & (np.abs(hg.astype(np.int32) - h_ref.astype(np.int32)) == 1))), \
        np.argwhere(diff & ~sgn)[:5]
    assert diff.mean() < 1e-3, diff.mean()
    codes, bscale, rscale = q_got
    ref = orc.quantize_nvfp4v(h_ref)
    same = ~diff.any(1)
    assert same.mean() > 0.5
    assert np.array_equal(codes[same], ref[0][same])
    assert np.array_equal(bscale[same], ref[1][same])
    assert np.array_equal(rscale[same].view(np.uint32), ref[2][same].view(np.uint32))
    if (~same).any():
        r = np.nonzero(~same)[0]
        deq = orc.dequant_nvfp4v(codes[r], bscale[r], rscale[r])
        d_b = np.repeat(np.array([[orc.e4m3_value(int(b)) for b in rowb] for rowb in bscale[r]]), 16, axis=1) \
            * rscale[r][:, None].astype(np.float64)
        href = bf16_bits_to_f32(h_ref[r]).astype(np.float64)
        hgot = bf16_bits_to_f32(hg[r]).astype(np.float64)
        # |x - q d_b| <= d_b (half the widest E2M1 gap; d_b itself is rounded to
        # binary32); a block whose scale byte underflows to 0 (d_b = 0) is all zero
        within = np.abs(deq - href) <= d_b * (1 + 1e-6) + np.abs(hgot - href)
        assert np.all(np.where(d_b == 0, deq == 0, within))


@pytest.mark.parametrize("rows,inter", [(1, 16), (37, 2048), (133, 1040), (64, 4096), (5, 16384)])
def test_swiglu_quantize_parity(orc, bsq_gpu, rows, inter):
    rng = rng_for(4, salt=inter + rows)
    gu = _gu(rng, rows, inter)
    h, codes, bscale, rscale = bsq_gpu.bsq_swiglu_quantize_nvfp4v(_dev(gu))
    _check(orc, bsq_gpu, gu, _np(h), (_np(codes), _np(bscale), _np(rscale)))


def test_swiglu_quantize_matches_standalone_quantizer(bsq_gpu):
    """The fused quantization of H gives the bytes the row quantizer gives for
    the H the kernel wrote; without an H output the codes are unchanged."""
    rng = rng_for(4, salt=7)
    gu = _dev(_gu(rng, 300, 2048))
    h, *q = bsq_gpu.bsq_swiglu_quantize_nvfp4v(gu)
    q2 = bsq_gpu.bsq_quantize_nvfp4v(h)
    _, *q3 = bsq_gpu.bsq_swiglu_quantize_nvfp4v(gu, write_h=False)
    for a, b, c in zip(q, q2, q3):
        a, b, c = _np(a), _np(b), _np(c)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        assert np.array_equal(a.view(np.uint8), c.view(np.uint8))


def test_swiglu_quantize_strided_and_edges(orc, bsq_gpu):
    """Strided gate/up rows (a column slice of a wider matrix), an all-zero
    row, zero gates (H = 0 exactly), huge negative gates (silu -> -0), gates
    whose e^-|g| is subnormal in binary32 and a sweep of gates over
    [-100, 100]."""
    rng = rng_for(4, salt=11)
    inter = 256
    wide = _gu(rng, 24, inter + 64)               # [24][2*inter + 128]
    wide[0] = 0
    wide[1, :inter] = 0
    wide[2, :inter] = f32_to_bf16_bits(np.full(inter, -200.0, np.float32))
    # gates where e^-|g| is below the binary32 normal range (|g| > 87.3) while
    # g e^g u is still a normal or subnormal bf16 value (moderate u: a huge u
    # would lift into range a product whose e^g binary32 cannot carry)
    wide[3, :inter] = f32_to_bf16_bits(np.linspace(-100.0, -80.0, inter).astype(np.float32))
    wide[3, inter:2 * inter] = f32_to_bf16_bits(np.linspace(0.5, 4.0, inter).astype(np.float32))
    wide[4, :inter] = f32_to_bf16_bits(np.linspace(-100.0, 100.0, inter).astype(np.float32))
    gu = np.ascontiguousarray(wide[:, :2 * inter])
    dev = _dev(wide)[:, :2 * inter]
    h, codes, bscale, rscale = bsq_gpu.bsq_swiglu_quantize_nvfp4v(dev)
    _check(orc, bsq_gpu, gu, _np(h), (_np(codes), _np(bscale), _np(rscale)))
    assert not _np(codes)[0].any() and _np(rscale)[0] == 0.0


def test_swiglu_quantize_full_size_sampled(orc, bsq_gpu):
    """The bench's shape (32768 token-slots x intermediate 2048) in one launch;
    the operation is row-local, so sampled rows are checked."""
    rng = rng_for(3, salt=13)
    M, inter = 32768, 2048
    gu = _gu(rng, M, inter)
    h, codes, bscale, rscale = bsq_gpu.bsq_swiglu_quantize_nvfp4v(_dev(gu))
    rows = np.unique(np.concatenate([np.arange(32), np.arange(M - 32, M), rng.choice(M, 192, replace=False)]))
    _check(orc, bsq_gpu, gu[rows], _np(h)[rows], (_np(codes)[rows], _np(bscale)[rows], _np(rscale)[rows]))


def test_swiglu_quantize_rejects_bad_shapes(bsq_gpu):
    gu = torch.zeros((4, 2 * 24), dtype=torch.bfloat16, device="cuda")   # inter = 24, not a multiple of 16
    with pytest.raises(RuntimeError):
        bsq_gpu.bsq_swiglu_quantize_nvfp4v(gu)
