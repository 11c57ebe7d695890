"""GPU parity of the gate/up grouped GEMM with SwiGLU in its epilogue
(bsq_grouped_gemm_fwd_swiglu), through the C ABI.

Against the unfused path (bsq_grouped_gemm_fwd writing gu in bf16, then
bsq_swiglu_quantize_nvfp4v): H bit for bit, and so the NVFP4v bytes of H.
Against the oracle: gu_ref = the float64 GEMM on the oracle's own quantized
operands, rounded to bf16 (the values the GEMM stores), and H_ref =
swiglu_bf16(gu_ref).  Where the GPU's bf16 gate and up values equal the
oracle's (all but elements whose float64 value sits next to a bf16 rounding
boundary), H lies within one bf16 ulp of H_ref (silu is evaluated in
binary32); rows whose H equals H_ref give the oracle's NVFP4v bytes exactly.
"""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, bf16_bits_to_f32, make_quantize_input, moe_counts, normal_bf16, \
    offsets_from_counts, rng_for

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def _h_vs_oracle(orc, h_bits, gu_gpu_bits, gu_ref_bits, inter):
    """One-ulp rule on the elements whose bf16 gate and up agree with the
    oracle's; returns the oracle's H and the mask of rows equal to it."""
    h_ref = orc.swiglu_bf16(gu_ref_bits)
    agree = (gu_gpu_bits[:, :inter] == gu_ref_bits[:, :inter]) & (gu_gpu_bits[:, inter:] == gu_ref_bits[:, inter:])
    assert agree.mean() > 0.99, agree.mean()
    hg = h_bits.view(np.uint16)
    diff = (hg != h_ref) & agree
    sgn = (hg >> 15) == (h_ref >> 15)
    one_ulp = np.abs(hg.astype(np.int32) - h_ref.astype(np.int32)) == 1
    assert np.all(~diff | (sgn & one_ulp)), np.argwhere(diff & ~(sgn & one_ulp))[:5]
    assert diff.sum() <= 1e-3 * agree.sum(), diff.mean()
    return h_ref, (hg == h_ref).all(1)


@pytest.mark.parametrize("counts,inter,k", [
    ([300, 0, 17, 1, 256, 513], 128, 256),      # ragged, empty, one-token experts, several row tiles
    ([129, 255, 257], 256, 448),                # two column tiles, k % 128 == 64 tail stage
    ([1000], 384, 1024),                        # one expert, three column tiles
    ([513, 2, 260], 128, 768),                  # three super-stages: the next tile fetched ahead
    ([128, 384, 129, 1], 128, 768),             # tails of 128 and 1 rows (half-height loop), 129 (full)
])
def test_gemm_swiglu_parity(orc, bsq_gpu, counts, inter, k):
    rng = rng_for(3, salt=inter + k)
    off = offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    x = make_quantize_input(rng, M, k)
    w = normal_bf16(rng, (E * 2 * inter, k), 0.05)
    a_q, w_q = orc.quantize_nvfp4v(x), orc.quantize_nvfp4v(w)
    a_d, w_d = bsq_gpu.bsq_quantize_nvfp4v(_dev(x.view(np.int16))), bsq_gpu.bsq_quantize_nvfp4v(_dev(w.view(np.int16)))
    for r, g in zip(a_q + w_q, a_d + w_d):
        assert np.array_equal(r.view(np.uint8), _np(g).view(np.uint8))
    offd = _dev(off)
    h_f = bsq_gpu.bsq_grouped_gemm_fwd_swiglu(a_d, w_d, offd, inter, k)
    gu = bsq_gpu.bsq_grouped_gemm_fwd(a_d, w_d, offd, 2 * inter, k)          # bf16 [gate | up]
    h_u, *q_u = bsq_gpu.bsq_swiglu_quantize_nvfp4v(gu)
    q_f = bsq_gpu.bsq_quantize_nvfp4v(h_f)
    assert np.array_equal(_np(h_f), _np(h_u))                               # the fused epilogue = the composition
    for a, b in zip(q_f, q_u):
        assert np.array_equal(_np(a).view(np.uint8), _np(b).view(np.uint8))
    gu_ref = orc.round_bf16(orc.grouped_gemm_fwd(a_q, w_q, off))
    h_ref, same = _h_vs_oracle(orc, _np(h_f), _np(gu).view(np.uint16), gu_ref, inter)
    assert same.mean() > 0.5
    ref = orc.quantize_nvfp4v(h_ref[same])
    for r, g in zip(ref, q_f):
        assert np.array_equal(r.view(np.uint8), _np(g)[same].view(np.uint8))


def test_gemm_swiglu_strided_output(bsq_gpu):
    """H written into a column slice of a wider matrix (ld_h > inter): same
    values, the other columns untouched."""
    rng = rng_for(3, salt=5)
    counts, inter, k = [70, 200], 128, 192
    off = offsets_from_counts(counts)
    M = int(off[-1])
    x, w = make_quantize_input(rng, M, k), normal_bf16(rng, (2 * 2 * inter, k), 0.05)
    a_d, w_d = bsq_gpu.bsq_quantize_nvfp4v(_dev(x.view(np.int16))), bsq_gpu.bsq_quantize_nvfp4v(_dev(w.view(np.int16)))
    h = bsq_gpu.bsq_grouped_gemm_fwd_swiglu(a_d, w_d, _dev(off), inter, k)
    wide = torch.full((M, inter + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    bsq_gpu.bsq_grouped_gemm_fwd_swiglu(a_d, w_d, _dev(off), inter, k, h=wide[:, 32:32 + inter])
    assert np.array_equal(_np(wide[:, 32:32 + inter]), _np(h))
    assert bool((wide[:, :32] == 7.0).all()) and bool((wide[:, 32 + inter:] == 7.0).all())


@pytest.mark.parametrize("cfg_id", [3, 5])
def test_gemm_swiglu_full_size(orc, bsq_gpu, cfg_id):
    """The bench's launch at full size (config 3: 32 experts, 32768 slots;
    config 5: 48 experts, 8 empty, 65536 slots; hidden 7168, intermediate
    2048): H equals the unfused path's everywhere, and sampled rows of six
    experts (smallest, largest and four more) satisfy the oracle rule."""
    cfg = CONFIGS[cfg_id]
    counts = moe_counts(cfg)
    off = offsets_from_counts(counts)
    E, I, Hd, M = cfg.n_experts, cfg.inter, cfg.hidden, cfg.m_total
    gen = torch.Generator(device="cuda").manual_seed(3030 + cfg_id)
    x = torch.randn((M, Hd), generator=gen, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E * 2 * I, Hd), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    a_d, w_d = bsq_gpu.bsq_quantize_nvfp4v(x), bsq_gpu.bsq_quantize_nvfp4v(w)
    offd = _dev(off)
    h_f = bsq_gpu.bsq_grouped_gemm_fwd_swiglu(a_d, w_d, offd, I, Hd)
    gu = bsq_gpu.bsq_grouped_gemm_fwd(a_d, w_d, offd, 2 * I, Hd)
    h_u, *_ = bsq_gpu.bsq_swiglu_quantize_nvfp4v(gu)
    assert torch.equal(h_f.view(torch.int16), h_u.view(torch.int16))
    del h_u
    rng = rng_for(cfg_id, salt=29)
    live = [int(e) for e in np.argsort(counts, kind="stable") if counts[e] > 0]
    picks = sorted({live[0], live[-1], *[live[i] for i in rng.choice(len(live), 4, replace=False)]})
    for e in picks:
        m0, m1 = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[m0, m1 - 1], rng.integers(m0, m1, 14)]))
        r_d = torch.from_numpy(rows).cuda()
        xa = _np(x[r_d]).view(np.uint16)
        we = _np(w[e * 2 * I:(e + 1) * 2 * I]).view(np.uint16)
        a_q, w_q = orc.quantize_nvfp4v(xa), orc.quantize_nvfp4v(we)
        gu_ref = orc.round_bf16(orc.grouped_gemm_fwd(a_q, w_q, np.array([0, len(rows)], np.int32)))
        _h_vs_oracle(orc, _np(h_f[r_d]), _np(gu[r_d]).view(np.uint16), gu_ref, I)
