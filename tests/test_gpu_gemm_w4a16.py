"""GPU parity of the frozen-expert grouped GEMM (bsq_grouped_gemm_w4a16: bf16
activations against NVFP4-variant packed weights dequantized in the kernel)
through the C ABI against the oracle's float64 product.  The weights' packed
bytes are checked equal between the GPU quantizer and the oracle's, and the
GEMM is compared on the oracle's bytes.  Every dequantized weight is exact in
bf16, products are exact in fp32 and accumulate in fp32, so the forward's
element-wise bound applies (module docstring of test_gpu_gemm); bf16 outputs
are the RNE of the kernel's own fp32 values."""
import numpy as np
import pytest
import torch

from test_gpu_gemm import _bf16_dev, _bits, _np, _sampled_rows, _to_dev, bf16_rne, check_groups
from test_oracle_gemm import packed_exact_weights
from workloads import CONFIGS, f32_to_bf16_bits, make_quantize_input, moe_counts, normal_bf16, offsets_from_counts, rng_for

pytestmark = pytest.mark.gpu


def _quantize_both(orc, bsq, w):
    w_q = orc.quantize_nvfp4v(w)
    w_d = bsq.bsq_quantize_nvfp4v(_bf16_dev(w))
    for r, g in zip(w_q, w_d):
        assert np.array_equal(r.view(np.uint8), _np(g).view(np.uint8))
    return w_q, w_d


def _case(orc, bsq, counts, n, k, seed):
    rng = rng_for(3, salt=seed)
    off = offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    x = make_quantize_input(rng, M, k)
    w = normal_bf16(rng, (E * n, k), 0.02)
    w_q, w_d = _quantize_both(orc, bsq, w)
    offd = _to_dev(off)
    y32 = bsq.bsq_grouped_gemm_w4a16(_bf16_dev(x), w_d, offd, n, k, y_dtype=bsq.BSQ_F32)
    y16 = bsq.bsq_grouped_gemm_w4a16(_bf16_dev(x), w_d, offd, n, k)
    ref = orc.grouped_gemm_w4a16(x, w_q, off)
    y32n = _np(y32)
    check_groups(y32n.astype(np.float64), ref, [(f"expert{e}", np.arange(off[e], off[e + 1])) for e in range(E)])
    assert np.array_equal(_bits(y16), bf16_rne(y32n))
    return y32n


@pytest.mark.parametrize("counts,n,k", [
    ([300, 0, 17, 1, 256, 513], 256, 256),
    ([1000], 512, 1024),
    ([40, 70, 9], 320, 64),
    ([129, 255, 257], 128, 448),
    ([3, 600], 64, 7168),
])
def test_w4a16_parity(orc, bsq_gpu, counts, n, k):
    """Ragged experts (empty, one-row, partial 256-row tiles), output widths
    that end inside a tile, and reductions of 1 to 112 super-stages."""
    _case(orc, bsq_gpu, counts, n, k, seed=3 * n + k)


def test_w4a16_exact_on_representable_weights(orc, bsq_gpu):
    """Weights the packed format holds exactly (row scale 1, power-of-two block
    scales) and integer activations: every partial sum is a multiple of 1/2
    below 2^22, so the kernel's fp32 result must equal the exact product."""
    rng = np.random.default_rng(41)
    counts = [100, 0, 260, 1]
    E, n, k = len(counts), 192, 256
    off = offsets_from_counts(counts)
    M = int(off[-1])
    wb, wv = packed_exact_weights(rng, E * n, k, jlo=0, jhi=3)
    w_q, w_d = _quantize_both(orc, bsq_gpu, wb)
    xi = rng.integers(-4, 5, (M, k)).astype(np.float64)
    y = _np(bsq_gpu.bsq_grouped_gemm_w4a16(_bf16_dev(f32_to_bf16_bits(xi.astype(np.float32))), w_d, _to_dev(off),
                                           n, k, y_dtype=bsq_gpu.BSQ_F32))
    for e in range(E):
        m0, m1 = int(off[e]), int(off[e + 1])
        assert np.array_equal(y[m0:m1].astype(np.float64), xi[m0:m1] @ wv[e * n:(e + 1) * n].T)


def test_w4a16_deterministic(orc, bsq_gpu):
    a = _case(orc, bsq_gpu, [200, 333, 0, 90], 256, 256, seed=19)
    b = _case(orc, bsq_gpu, [200, 333, 0, 90], 256, 256, seed=19)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_w4a16_full_size_sampled(orc, bsq_gpu, which):
    """The 32-expert shapes in one launch (as the bench runs them); sampled
    rows of every expert and sampled output columns, the weight rows' packed
    bytes checked against the oracle's quantizer."""
    cfg = CONFIGS[3]
    counts = moe_counts(cfg)
    off = offsets_from_counts(counts)
    E, M = cfg.n_experts, cfg.m_total
    n, k = (2 * cfg.inter, cfg.hidden) if which == "gate_up" else (cfg.hidden, cfg.inter)
    gen = torch.Generator(device="cuda").manual_seed(7007 + n)
    x = torch.randn((M, k), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E * n, k), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    w_d = bsq_gpu.bsq_quantize_nvfp4v(w)
    y = bsq_gpu.bsq_grouped_gemm_w4a16(x, w_d, _to_dev(off), n, k, y_dtype=bsq_gpu.BSQ_F32)
    rng = rng_for(3, salt=31)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    colsd = torch.from_numpy(cols).cuda()
    for e, rows in _sampled_rows(off, rng, 2, 2, 4):
        xr = _bits(x[torch.from_numpy(rows).cuda()])
        wr = _bits(w[e * n:(e + 1) * n][colsd])
        w_q = orc.quantize_nvfp4v(wr)
        for r, g in zip(w_q, w_d):
            assert np.array_equal(r.view(np.uint8), _np(g[e * n:(e + 1) * n][colsd]).view(np.uint8))
        ref = orc.grouped_gemm_w4a16(xr, w_q, np.array([0, len(rows)], np.int32))
        got = _np(y[torch.from_numpy(rows).cuda()][:, colsd]).astype(np.float64)
        check_groups(got, ref, [((which, e), np.arange(len(rows)))])


@pytest.mark.parametrize("E", [200, 900])
def test_w4a16_many_experts(orc, bsq_gpu, E):
    """Many small experts, a third of them empty: tile decode from the LDS
    tables (200) and from the planner's arrays in global memory (900)."""
    rng = rng_for(7, salt=E + 3)
    counts = rng.integers(0, 24, E)
    counts[rng.random(E) < 0.33] = 0
    _case(orc, bsq_gpu, list(counts), 64, 128, seed=E + 5)
