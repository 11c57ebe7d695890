"""Fast-divide ablation of the NVFP4-variant quantizer on the GPU
(bsq_debug_quantize_nvfp4v_fastdiv): every division replaced by the hardware
reciprocal approximation times the numerator.  The bytes cannot be pinned
exactly (the reciprocal's rounding is not specified beyond its error bound),
so the test checks what the bound implies: the divide's relative error is a
few ulps (below 2^-20), so against the exact-division quantization from the
oracle a block scale may differ only where 448 a_b / A lies within 2^-20 of
an E4M3 rounding boundary, a code only where x / d_b lies within 2^-20 of an
E2M1 boundary (in blocks whose scale did not change), and a changed code is
a neighbour on the E2M1 grid."""
import numpy as np
import pytest
import torch

from workloads import make_quantize_input, rng_for

pytestmark = pytest.mark.gpu
DELTA = 2.0 ** -20


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_fastdiv_changes_only_boundary_decisions(orc, bsq_gpu):
    rng = rng_for(2, salt=77)
    x = make_quantize_input(rng, 1024, 7168)
    codes, bscale, rscale = orc.quantize_nvfp4v(x)
    fc, fb, fr = (_np(t) for t in bsq_gpu.bsq_debug_quantize_nvfp4v_fastdiv(
        torch.from_numpy(x.view(np.int16)).cuda()))
    blocks, elems = orc.nvfp4v_decision_margins(x, DELTA)
    # row scales: A / 2688 within a few ulps
    assert np.all(np.abs(fr.astype(np.float64) / rscale.astype(np.float64) - 1) <= 2.0 ** -21)
    sb_changed = fb != bscale
    assert not (sb_changed & ~blocks).any()
    nib = lambda c: np.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1)
    cn, fn = nib(codes), nib(fc)
    changed = cn != fn
    same_block = np.repeat(~sb_changed, 16, axis=1)
    assert not (changed & same_block & ~elems).any()
    # a changed code moves to a neighbouring E2M1 magnitude (or flips only the sign of a zero)
    ch = changed & same_block
    mag_a, mag_b = cn[ch] & 7, fn[ch] & 7
    zero_sign = (mag_a == 0) & (mag_b == 0)
    assert np.all(zero_sign | ((np.abs(mag_a.astype(int) - mag_b.astype(int)) == 1) & ((cn[ch] >> 3) == (fn[ch] >> 3))))


def test_fastdiv_rejects_like_the_quantizer(bsq_gpu):
    with pytest.raises(RuntimeError):
        bsq_gpu.bsq_debug_quantize_nvfp4v_fastdiv(torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda"))
