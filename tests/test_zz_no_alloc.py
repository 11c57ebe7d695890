"""The allocation-free forward GEMM entry point against the workspace one:
bit-identical outputs on two calls in a row, the second with fewer experts
and rows than the first (the library's device array then still holds the
first call's planner tables)."""
import numpy as np
import pytest
import torch

from workloads import make_quantize_input, normal_bf16, offsets_from_counts, rng_for

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(bsq, counts, n, k, seed):
    rng = rng_for(6, salt=seed)
    off = offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    x = make_quantize_input(rng, M, k)
    w = normal_bf16(rng, (E * n, k), 0.02)
    a_d = bsq.bsq_quantize_nvfp4v(_dev(x.view(np.int16)))
    w_d = bsq.bsq_quantize_nvfp4v(_dev(w.view(np.int16)))
    return a_d, w_d, _dev(off)


def test_noalloc_matches_workspace_entry(bsq_gpu):
    rng = rng_for(6, salt=1)
    big = list(rng.integers(0, 90, 200))
    big[3] = 0
    big[17] = 700
    cases = [(big, 512, 1024, 1), ([40, 0, 70, 9], 264, 256, 2)]   # second call: fewer experts and rows
    for counts, n, k, seed in cases:
        a_d, w_d, offd = _case(bsq_gpu, counts, n, k, seed)
        for dt in (bsq_gpu.BSQ_F32, bsq_gpu.BSQ_BF16):
            ref = bsq_gpu.bsq_grouped_gemm_fwd(a_d, w_d, offd, n, k, y_dtype=dt)
            got = bsq_gpu.bsq_grouped_gemm_fwd_noalloc(a_d, w_d, offd, n, k, y_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(ref.view(torch.int16 if dt == bsq_gpu.BSQ_BF16 else torch.int32),
                               got.view(torch.int16 if dt == bsq_gpu.BSQ_BF16 else torch.int32)), (len(counts), dt)


def test_noalloc_rejects_too_many_experts(bsq_gpu):
    a_d, w_d, _ = _case(bsq_gpu, [64], 64, 128, 3)
    off = torch.zeros(4098, dtype=torch.int32, device="cuda")
    off[-1] = 64
    with pytest.raises(bsq_gpu.BsqError) as ei:
        bsq_gpu.bsq_grouped_gemm_fwd_noalloc(a_d, (w_d[0].repeat(4097, 1), w_d[1].repeat(4097, 1),
                                                   w_d[2].repeat(4097)), off, 64, 128)
    assert ei.value.status == bsq_gpu.BSQ_ERR_UNSUPPORTED
