"""GPU parity of the all-MXFP8 forward grouped GEMM (bsq_grouped_gemm_fwd_mxfp8)
through the C ABI against the oracle's float64 product of the dequantized
operands.  It runs on the block-scaled fp8 MFMA, so it is held to the same
bounds as the backward GEMMs (module docstring of test_gpu_gemm): per expert
max |y - r| / max |r| <= 2e-3 and |y - r| <= 2^-11 * sum_k |x_k w_k| element by
element; bf16 outputs are the RNE of the kernel's own fp32 values.  The
operands handed to the oracle are quantized by the oracle from the same bf16
inputs, after asserting the GPU quantizer produced the same bytes."""
import numpy as np
import pytest
import torch

from test_gpu_gemm import _bf16_dev, _bits, _np, _sampled_rows, _to_dev, bf16_rne, check_groups
from workloads import CONFIGS, make_quantize_input, moe_counts, normal_bf16, offsets_from_counts, rng_for

pytestmark = pytest.mark.gpu


def _case(orc, bsq, counts, n, k, seed):
    rng = rng_for(3, salt=seed)
    off = offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    x = make_quantize_input(rng, M, k)
    w = normal_bf16(rng, (E * n, k), 0.02)
    x_q, w_q = orc.quantize_mxfp8_rowwise(x), orc.quantize_mxfp8_rowwise(w)
    x_d = bsq.bsq_quantize_mxfp8(_bf16_dev(x), bsq.BSQ_ROWWISE)
    w_d = bsq.bsq_quantize_mxfp8(_bf16_dev(w), bsq.BSQ_ROWWISE)
    for r, g in zip(x_q + w_q, x_d + w_d):
        assert np.array_equal(r, _np(g))
    offd = _to_dev(off)
    y32 = bsq.bsq_grouped_gemm_fwd_mxfp8(x_d, w_d, offd, n, k, y_dtype=bsq.BSQ_F32)
    y16 = bsq.bsq_grouped_gemm_fwd_mxfp8(x_d, w_d, offd, n, k)
    ref = orc.grouped_gemm_fwd_mxfp8(x_q, w_q, off)
    absum = orc.grouped_gemm_fwd_mxfp8(x_q, w_q, off, absolute=True)
    y32n = _np(y32)
    check_groups(y32n.astype(np.float64), ref, [(f"expert{e}", np.arange(off[e], off[e + 1])) for e in range(E)],
                 strict=False, absum=absum)
    assert np.array_equal(_bits(y16), bf16_rne(y32n))
    return y32n


@pytest.mark.parametrize("counts,n,k", [
    ([300, 0, 17, 1, 256, 513], 256, 256),      # ragged, empty, one-token experts, several tiles
    ([1000], 512, 1024),                        # one expert = dense GEMM
    ([40, 70, 9], 320, 64),                     # n not a tile multiple, k = one k step
    ([129, 255, 257], 128, 448),                # k % 128 == 64: half a super-stage at the end
])
def test_fwd_mxfp8_parity(orc, bsq_gpu, counts, n, k):
    _case(orc, bsq_gpu, counts, n, k, seed=n + 3 * k)


def test_fwd_mxfp8_deterministic(orc, bsq_gpu):
    a = _case(orc, bsq_gpu, [200, 333, 0, 90], 256, 256, seed=5)
    b = _case(orc, bsq_gpu, [200, 333, 0, 90], 256, 256, seed=5)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_fwd_mxfp8_full_size_sampled(orc, bsq_gpu, which):
    """The 32-expert shard (32768 token-slots, Zipf(1.1)) at the bench's
    shapes, one launch; sampled rows of every expert and sampled output
    columns are checked against the oracle."""
    cfg = CONFIGS[3]
    counts = moe_counts(cfg)
    off = offsets_from_counts(counts)
    E, M = cfg.n_experts, cfg.m_total
    n, k = (2 * cfg.inter, cfg.hidden) if which == "gate_up" else (cfg.hidden, cfg.inter)
    gen = torch.Generator(device="cuda").manual_seed(5005 + n)
    x = torch.randn((M, k), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E * n, k), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    offd = _to_dev(off)
    x_d = bsq_gpu.bsq_quantize_mxfp8(x, bsq_gpu.BSQ_ROWWISE)
    w_d = bsq_gpu.bsq_quantize_mxfp8(w, bsq_gpu.BSQ_ROWWISE)
    y = bsq_gpu.bsq_grouped_gemm_fwd_mxfp8(x_d, w_d, offd, n, k, y_dtype=bsq_gpu.BSQ_F32)
    rng = rng_for(3, salt=23)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    colsd = torch.from_numpy(cols).cuda()
    for e, rows in _sampled_rows(off, rng, 2, 2, 4):
        x_q = orc.quantize_mxfp8_rowwise(_bits(x[torch.from_numpy(rows).cuda()]))
        w_q = orc.quantize_mxfp8_rowwise(_bits(w[e * n:(e + 1) * n][colsd]))
        seg = np.array([0, len(rows)], np.int32)
        ref = orc.grouped_gemm_fwd_mxfp8(x_q, w_q, seg)
        absum = orc.grouped_gemm_fwd_mxfp8(x_q, w_q, seg, absolute=True)
        got = _np(y[torch.from_numpy(rows).cuda()][:, colsd]).astype(np.float64)
        check_groups(got, ref, [((which, e), np.arange(len(rows)))], strict=False, absum=absum)


def test_fwd_mxfp8_rejects_unsupported(bsq_gpu):
    x = bsq_gpu.bsq_quantize_mxfp8(torch.zeros((8, 96), dtype=torch.bfloat16, device="cuda"), bsq_gpu.BSQ_ROWWISE)
    w = bsq_gpu.bsq_quantize_mxfp8(torch.zeros((2 * 64, 96), dtype=torch.bfloat16, device="cuda"),
                                   bsq_gpu.BSQ_ROWWISE)
    off = _to_dev(np.array([0, 4, 8], np.int32))
    with pytest.raises(RuntimeError):   # k = 96 is not a multiple of 64
        bsq_gpu.bsq_grouped_gemm_fwd_mxfp8(x, w, off, 64, 96)
