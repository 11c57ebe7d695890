"""GPU parity of the bf16 baseline grouped GEMM (bsq_grouped_gemm_bf16)
through the C ABI against the oracle's float64 product of the same bf16
inputs.  bf16 products are exact in fp32 and accumulate in fp32, so the
forward's element-wise bound applies (module docstring of test_gpu_gemm):
per expert max |y - r| / max(|r|, 0.01 rms) <= 2e-3; bf16 outputs are the RNE
of the kernel's own fp32 values."""
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
    offd = _to_dev(off)
    y32 = bsq.bsq_grouped_gemm_bf16(_bf16_dev(x), _bf16_dev(w), offd, n, k, y_dtype=bsq.BSQ_F32)
    y16 = bsq.bsq_grouped_gemm_bf16(_bf16_dev(x), _bf16_dev(w), offd, n, k)
    ref = orc.grouped_gemm_bf16(x, w, off)
    y32n = _np(y32)
    check_groups(y32n.astype(np.float64), ref, [(f"expert{e}", np.arange(off[e], off[e + 1])) for e in range(E)])
    assert np.array_equal(_bits(y16), bf16_rne(y32n))
    return y32n


@pytest.mark.parametrize("counts,n,k", [
    ([300, 0, 17, 1, 256, 513], 256, 256),
    ([1000], 512, 1024),
    ([40, 70, 9], 320, 64),
    ([129, 255, 257], 128, 448),
])
def test_bf16_gemm_parity(orc, bsq_gpu, counts, n, k):
    _case(orc, bsq_gpu, counts, n, k, seed=2 * n + k)


def test_bf16_gemm_deterministic(orc, bsq_gpu):
    a = _case(orc, bsq_gpu, [200, 333, 0, 90], 256, 256, seed=9)
    b = _case(orc, bsq_gpu, [200, 333, 0, 90], 256, 256, seed=9)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_bf16_gemm_full_size_sampled(orc, bsq_gpu, which):
    """The bench's 32-expert shapes in one launch; sampled rows of every
    expert and sampled output columns."""
    cfg = CONFIGS[3]
    counts = moe_counts(cfg)
    off = offsets_from_counts(counts)
    E, M = cfg.n_experts, cfg.m_total
    n, k = (2 * cfg.inter, cfg.hidden) if which == "gate_up" else (cfg.hidden, cfg.inter)
    gen = torch.Generator(device="cuda").manual_seed(6006 + n)
    x = torch.randn((M, k), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E * n, k), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    y = bsq_gpu.bsq_grouped_gemm_bf16(x, w, _to_dev(off), n, k, y_dtype=bsq_gpu.BSQ_F32)
    rng = rng_for(3, salt=29)
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    colsd = torch.from_numpy(cols).cuda()
    for e, rows in _sampled_rows(off, rng, 2, 2, 4):
        xr = _bits(x[torch.from_numpy(rows).cuda()])
        we = _bits(w[e * n:(e + 1) * n][colsd])
        ref = orc.grouped_gemm_bf16(xr, we, np.array([0, len(rows)], np.int32))
        got = _np(y[torch.from_numpy(rows).cuda()][:, colsd]).astype(np.float64)
        check_groups(got, ref, [((which, e), np.arange(len(rows)))])
