"""GPU parity of the quantizers through the C ABI: bit-exact codes, scale
bytes and per-row fp32 scales against the CPU oracle on the same seeded bf16
inputs, plus exhaustive sweeps of the device element encoders."""
import numpy as np
import pytest
import torch

from conftest import bf16
from workloads import (bf16_bits_to_f32, make_quantize_input, normal_bf16, offsets_from_counts, rng_for,
                       expert_counts_zipf)

pytestmark = pytest.mark.gpu


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bf16_dev(bits):
    return _to_dev(bits.view(np.int16))


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------ exhaustive encoders

def _breakpoints(encode, max_code):
    """First fp32 bit pattern (>= 0) of each code of a monotone encoder, from
    the oracle, by binary search over the non-negative bit patterns."""
    def code_at(u):
        return int(encode(np.array([u], np.uint32).view(np.float32))[0])
    starts = [0]
    codes = [code_at(0)]
    lo_u = 0
    while codes[-1] != max_code:
        c = codes[-1]
        lo, hi = lo_u, 0x7F800000  # code_at(hi) == max_code (inf saturates)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if code_at(mid) > c:
                hi = mid
            else:
                lo = mid
        starts.append(hi)
        codes.append(code_at(hi))
        lo_u = hi
    return np.array(starts, np.int64), np.array(codes, np.int64)


@pytest.mark.parametrize("which", ["e2m1", "e4m3"])
def test_encoder_exhaustive_all_fp32(orc, bsq_gpu, which):
    """Every non-NaN fp32 bit pattern, both signs, through the device encoder
    the quantizers use, against runs derived from the oracle's encoder."""
    if which == "e2m1":
        enc, dev_enc, max_code, sign = orc.e2m1_encode, bsq_gpu.bsq_debug_encode_e2m1, 7, 8
    else:
        enc, dev_enc, max_code, sign = orc.e4m3_encode, bsq_gpu.bsq_debug_encode_e4m3, 0x7E, 0x80
    starts, codes = _breakpoints(enc, max_code)
    # monotone encoder: the runs are the whole truth (spot check them)
    probe = np.concatenate([starts, np.maximum(starts - 1, 0)]).astype(np.uint32)
    ref_probe = np.searchsorted(starts, probe.astype(np.int64), side="right") - 1
    assert np.array_equal(enc(probe.view(np.float32)), codes[ref_probe].astype(np.uint8))
    top = 0x7F800001  # +inf included, NaNs excluded
    chunk = 1 << 27
    starts_d = torch.from_numpy(starts).cuda()
    codes_d = torch.from_numpy(codes).cuda().to(torch.uint8)
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    bad = 0
    for s_bit in (0, 1 << 31):
        for lo in range(0, top, chunk):
            n = min(chunk, top - lo)
            u = torch.arange(lo, lo + n, dtype=torch.int64, device="cuda")
            v = u | s_bit                                   # unsigned 32-bit pattern
            x = torch.where(v >= (1 << 31), v - (1 << 32), v).to(torch.int32).view(torch.float32)
            dev_enc(x, out[:n])
            idx = torch.searchsorted(starts_d, u, right=True) - 1
            exp = codes_d[idx] | (sign if s_bit else 0)
            bad += int((out[:n] != exp).sum())
    assert bad == 0


# ------------------------------------------------------------ NVFP4 variant

def _nvfp4v_check(orc, bsq_gpu, x_bits):
    ref = orc.quantize_nvfp4v(x_bits)
    got = bsq_gpu.bsq_quantize_nvfp4v(_bf16_dev(x_bits))
    for r, g, nm in zip(ref, got, ("codes", "bscale", "rscale")):
        g = _np(g)
        if nm == "rscale":
            assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), nm
        else:
            assert np.array_equal(r, g), (nm, np.argwhere(r != g)[:5])


@pytest.mark.parametrize("cols", [16, 48, 256, 2048, 7168, 16384])
def test_nvfp4v_parity_shapes(orc, bsq_gpu, cols):
    rng = rng_for(2, salt=cols)
    rows = 37 if cols >= 7168 else 133
    _nvfp4v_check(orc, bsq_gpu, make_quantize_input(rng, rows, cols))


def test_nvfp4v_parity_edge_values(orc, bsq_gpu):
    rng = rng_for(2, salt=99)
    x = normal_bf16(rng, (24, 256))
    x[0] = 0                                     # zero row
    x[1] = bf16(np.full(256, -0.0))              # negative-zero row
    x[2, :16] = 0                                # zero block
    x[3] = bf16(rng.standard_normal(256) * 2.0 ** 120)   # 448*a_b overflow path
    x[4] = bf16(rng.standard_normal(256) * 2.0 ** -128)  # subnormal bf16 values
    x[5, :] = bf16(np.full(256, 2.0 ** -133))    # smallest subnormal everywhere
    x[6] = bf16(np.where(rng.random(256) < 0.5, 3.0e38, -1e-30))
    golden = [2688, -1344, 112, 336, 560, 784, 1120, 1568, 2240, -56, 0, 1, -2688, 200, -200, 100]
    x[7, :16] = bf16(golden)                     # every E2M1 tie
    x[7, 16:] = bf16(np.tile(golden, 15) * 0.75)
    x[8] = bf16(rng.standard_normal(256) * 2.0 ** -100)
    x[9, ::16] = bf16(np.full(16, 1.0))          # one nonzero per block
    x[9, 1::16] = bf16(np.full(16, 2.0 ** -12))
    x[10] = bf16(rng.integers(-6, 7, 256) * 0.5)
    # block maxima in [FLT_MAX / 1.75, bf16 max] = [1.94e38, 3.39e38]: the
    # branch where 448 * a_b would overflow binary32
    top = rng.uniform(1.95e38, 3.38e38, 16)
    x[11] = bf16(np.repeat(top, 16) * rng.uniform(-1, 1, 256))
    x[11, ::16] = bf16(top)
    x[12] = bf16(np.tile([1.75 * 2.0 ** 127, 1.25 * 2.0 ** 127], 128) * np.repeat([1, -1], 128))
    for r in range(13, 24):
        xf = bf16_bits_to_f32(x[r]).astype(np.float64)
        xf = xf if not np.abs(xf).max() else xf * 2.0 ** (127 - np.floor(np.log2(np.abs(xf).max())))
        x[r] = bf16(xf)
    _nvfp4v_check(orc, bsq_gpu, x)


def test_nvfp4v_full_size_sampled_rows(orc, bsq_gpu):
    """Config 2 at full size (16384 x 7168, outlier channels) in one launch;
    the quantizer is row-local, so sampled rows are checked exactly."""
    rng = rng_for(2)
    x = make_quantize_input(rng, 16384, 7168)
    got = bsq_gpu.bsq_quantize_nvfp4v(_bf16_dev(x))
    rows = np.unique(np.concatenate([np.arange(64), np.arange(16384 - 64, 16384),
                                     rng.choice(16384, 256, replace=False)]))
    ref = orc.quantize_nvfp4v(x[rows])
    for r, g in zip(ref, got):
        assert np.array_equal(r.view(np.uint8), _np(g)[rows].view(np.uint8))


def test_nvfp4v_batch_invariance_gpu(bsq_gpu):
    """A row quantized in any batch (shuffled, random batch sizes) gives the
    same bytes: per-token scaling, no tensor-wide statistic."""
    rng = rng_for(5, salt=3)
    x = make_quantize_input(rng, 2048, 7168)
    xd = _bf16_dev(x)
    full = [_np(t) for t in bsq_gpu.bsq_quantize_nvfp4v(xd)]
    for _ in range(16):
        n = int(rng.integers(1, 2048))
        sel = rng.permutation(2048)[:n]
        part = bsq_gpu.bsq_quantize_nvfp4v(xd[torch.from_numpy(sel).cuda()].contiguous())
        for f, p in zip(full, part):
            assert np.array_equal(f[sel].view(np.uint8), _np(p).view(np.uint8))


def test_mxfp8_rowwise_batch_invariance_gpu(bsq_gpu):
    """MXFP8 row-wise codes and scale bytes of a row do not depend on the
    batch it is quantized in (shuffled batches of random sizes)."""
    rng = rng_for(5, salt=4)
    x = make_quantize_input(rng, 1024, 7168)
    xd = _bf16_dev(x)
    fc, fs = [_np(t) for t in bsq_gpu.bsq_quantize_mxfp8(xd, bsq_gpu.BSQ_ROWWISE)]
    for _ in range(16):
        n = int(rng.integers(1, 1024))
        sel = rng.permutation(1024)[:n]
        pc, ps = bsq_gpu.bsq_quantize_mxfp8(xd[torch.from_numpy(sel).cuda()].contiguous(), bsq_gpu.BSQ_ROWWISE)
        assert np.array_equal(fc[sel], _np(pc)) and np.array_equal(fs[:, sel], _np(ps))


def test_nvfp4v_strided_input(orc, bsq_gpu):
    rng = rng_for(2, salt=5)
    big = make_quantize_input(rng, 40, 512)
    xd = _bf16_dev(big)[:, 128:384]
    got = bsq_gpu.bsq_quantize_nvfp4v(xd)
    ref = orc.quantize_nvfp4v(np.ascontiguousarray(big[:, 128:384]))
    for r, g in zip(ref, got):
        assert np.array_equal(r.view(np.uint8), _np(g).view(np.uint8))


# ------------------------------------------------------------------ MXFP8

@pytest.mark.parametrize("rows,cols", [(129, 32), (129, 96), (129, 2048), (129, 7168), (384, 1056), (16, 7168)])
def test_mxfp8_rowwise_parity(orc, bsq_gpu, rows, cols):
    """Row tiles of 128 rows and 1024 columns: partial row tiles, partial
    column tiles, and both scale write paths (16-byte runs when the row count
    is a multiple of 16, bytes otherwise)."""
    rng = rng_for(2, salt=100 + cols + rows)
    x = make_quantize_input(rng, rows, cols)
    x[0] = 0
    x[1, :32] = bf16(np.full(32, 2.0 ** -130))
    x[2] = bf16(rng.standard_normal(cols) * 2.0 ** 125)
    x[3] = bf16(rng.standard_normal(cols) * 1e-3)
    x[4, :32] = bf16(np.array([3.875, -0.0] + [0.5] * 30))
    rc, rs = orc.quantize_mxfp8_rowwise(x)
    gc, gs = bsq_gpu.bsq_quantize_mxfp8(_bf16_dev(x), bsq_gpu.BSQ_ROWWISE)
    assert np.array_equal(rc, _np(gc)) and np.array_equal(rs, _np(gs))


@pytest.mark.parametrize("case", ["ragged", "empty_groups", "single", "weights"])
def test_mxfp8_colwise_t_parity(orc, bsq_gpu, case):
    rng = rng_for(4, salt=["ragged", "empty_groups", "single", "weights"].index(case))
    if case == "ragged":
        counts = [37, 0, 300, 1, 64, 95, 33]
        cols = 264
    elif case == "empty_groups":
        counts = [0, 0, 70, 0, 0]
        cols = 96
    elif case == "single":
        counts = [1000]
        cols = 512
    else:  # expert weights [E][N][K] as rows E*N with offsets multiples of N
        counts = [128] * 4
        cols = 256
    off = offsets_from_counts(counts)
    M = int(off[-1])
    x = make_quantize_input(rng, M, cols) if M else np.zeros((0, cols), np.uint16)
    rc, rs = orc.quantize_mxfp8_colwise_t(x, off)
    gc, gs = bsq_gpu.bsq_quantize_mxfp8(_bf16_dev(x), bsq_gpu.BSQ_COLWISE_T, offsets=_to_dev(off))
    assert np.array_equal(rc, _np(gc)), np.argwhere(rc != _np(gc))[:5]
    assert np.array_equal(rs, _np(gs))


def test_mxfp8_colwise_t_full_size_sampled(orc, bsq_gpu):
    """dY-shaped input at full size (32768 x 7168, Zipf(1.1) over 32 experts):
    the transposed layout is checked exactly on sampled channels (columns are
    independent) for every expert segment, plus all padding bytes."""
    from workloads import CONFIGS, moe_counts
    counts = moe_counts(CONFIGS[4])
    off = offsets_from_counts(counts)
    gen = torch.Generator(device="cuda").manual_seed(1004)
    dy = (torch.randn((32768, 7168), generator=gen, device="cuda") * 1e-3).to(torch.bfloat16)
    gc, gs = bsq_gpu.bsq_quantize_mxfp8(dy, bsq_gpu.BSQ_COLWISE_T, offsets=_to_dev(off))
    rng = rng_for(4, salt=7)
    ch = np.unique(np.concatenate([[0, 7167], rng.choice(7168, 30, replace=False)]))
    x_ch = _np(dy[:, torch.from_numpy(ch).cuda()].contiguous().view(torch.int16)).view(np.uint16)
    rc, rs = orc.quantize_mxfp8_colwise_t(np.ascontiguousarray(x_ch), off)
    gcn = _np(gc[torch.from_numpy(ch).cuda()])
    gsn = _np(gs[:, torch.from_numpy(ch).cuda()])
    assert np.array_equal(rc, gcn) and np.array_equal(rs, gsn)


@pytest.mark.parametrize("counts,cols", [([37, 0, 300, 1, 64, 95, 33], 288), ([0, 0, 70, 0, 0], 96),
                                         ([1000], 512), ([128] * 4, 256), ([5, 250, 3], 2048)])
def test_mxfp8_dual_parity(orc, bsq_gpu, counts, cols):
    """One read, both layouts: the ROWWISE bytes and the per-group COLWISE_T
    bytes against the oracle's two quantizers, on ragged groups (empty ones,
    a one-token group, partial 32-blocks), partial channel tiles and the
    special values of the row-wise test."""
    rng = rng_for(4, salt=50 + cols + len(counts))
    off = offsets_from_counts(counts)
    M = int(off[-1])
    x = make_quantize_input(rng, M, cols)
    x[0] = 0
    x[1, :32] = bf16(np.full(32, 2.0 ** -130))
    x[2] = bf16(rng.standard_normal(cols) * 2.0 ** 125)
    x[3] = bf16(rng.standard_normal(cols) * 1e-3)
    x[4, :32] = bf16(np.array([3.875, -0.0] + [0.5] * 30))
    (grc, grs), (gtc, gts) = bsq_gpu.bsq_quantize_mxfp8_dual(_bf16_dev(x), _to_dev(off))
    rc, rs = orc.quantize_mxfp8_rowwise(x)
    tc, ts = orc.quantize_mxfp8_colwise_t(x, off)
    assert np.array_equal(rc, _np(grc)), np.argwhere(rc != _np(grc))[:5]
    assert np.array_equal(rs, _np(grs))
    assert np.array_equal(tc, _np(gtc)), np.argwhere(tc != _np(gtc))[:5]
    assert np.array_equal(ts, _np(gts))


@pytest.mark.parametrize("G", [200, 900])
def test_mxfp8_dual_many_groups(orc, bsq_gpu, G):
    """More than 61 groups (the segment lookup's wave-wide search path), a
    third of them empty, both layouts against the oracle."""
    rng = rng_for(4, salt=G)
    counts = rng.integers(0, 40, G)
    counts[rng.random(G) < 0.33] = 0
    off = offsets_from_counts(counts)
    M = int(off[-1])
    x = make_quantize_input(rng, M, 160)
    (grc, grs), (gtc, gts) = bsq_gpu.bsq_quantize_mxfp8_dual(_bf16_dev(x), _to_dev(off))
    rc, rs = orc.quantize_mxfp8_rowwise(x)
    tc, ts = orc.quantize_mxfp8_colwise_t(x, off)
    assert np.array_equal(rc, _np(grc)) and np.array_equal(rs, _np(grs))
    assert np.array_equal(tc, _np(gtc)) and np.array_equal(ts, _np(gts))


def test_mxfp8_dual_strided_full_size_sampled(orc, bsq_gpu):
    """dGU-shaped input at full size (32768 x 4096, Zipf(1.1) over 32 experts)
    read through a leading dimension wider than the row: sampled rows checked
    ROWWISE and sampled channels COLWISE_T against the oracle."""
    from workloads import CONFIGS, moe_counts
    counts = moe_counts(CONFIGS[4])
    off = offsets_from_counts(counts)
    gen = torch.Generator(device="cuda").manual_seed(1005)
    base = (torch.randn((32768, 4096 + 64), generator=gen, device="cuda") * 1e-3).to(torch.bfloat16)
    x = base[:, :4096]
    (grc, grs), (gtc, gts) = bsq_gpu.bsq_quantize_mxfp8_dual(x, _to_dev(off))
    rng = rng_for(4, salt=8)
    rows = np.unique(np.concatenate([[0, 32767], off[1:-1] - 1, rng.choice(32768, 60, replace=False)]))
    rows = rows[(rows >= 0) & (rows < 32768)]
    x_rows = _np(x[torch.from_numpy(rows).cuda()].contiguous().view(torch.int16)).view(np.uint16)
    rc, rs = orc.quantize_mxfp8_rowwise(x_rows)
    assert np.array_equal(rc, _np(grc)[rows]) and np.array_equal(rs, _np(grs)[:, rows])
    ch = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 24, replace=False)]))
    x_ch = _np(x[:, torch.from_numpy(ch).cuda()].contiguous().view(torch.int16)).view(np.uint16)
    tc, ts = orc.quantize_mxfp8_colwise_t(np.ascontiguousarray(x_ch), off)
    assert np.array_equal(tc, _np(gtc[torch.from_numpy(ch).cuda()]))
    assert np.array_equal(ts, _np(gts[:, torch.from_numpy(ch).cuda()]))


@pytest.mark.parametrize("src_rows,rows,cols", [(300, 300, 256), (97, 4 * 97, 1056), (64, 130, 7168)])
def test_mxfp8_gather_parity(orc, bsq_gpu, src_rows, rows, cols):
    """Dispatch-style permutation fused into the MXFP8 row-wise quantizer:
    repeated indices (top-k duplicates), a shuffled order and out-of-range
    indices (zero rows), against the oracle on the gathered rows."""
    rng = rng_for(2, salt=src_rows + cols)
    x = make_quantize_input(rng, src_rows, cols)
    idx = rng.integers(0, src_rows, rows).astype(np.int32)
    idx[:3] = [-1, src_rows, 2 ** 31 - 1]
    ref = orc.quantize_mxfp8_gather(x, idx)
    got = bsq_gpu.bsq_quantize_mxfp8_gather(_bf16_dev(x), _to_dev(idx))
    for r, g in zip(ref, got):
        assert np.array_equal(r, _np(g))


def test_mxfp8_gather_full_size_sampled(orc, bsq_gpu):
    """4096 tokens x 7168 dispatched with top-8 routing into 32768 expert-sorted
    slots in one launch; sampled output rows checked against the oracle."""
    rng = rng_for(3, salt=41)
    T, C, k, E = 4096, 7168, 8, 32
    x = make_quantize_input(rng, T, C)
    picks = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    order = np.argsort(picks.reshape(-1), kind="stable")
    idx = (order // k).astype(np.int32)            # slot -> token, expert-sorted
    codes, scale = bsq_gpu.bsq_quantize_mxfp8_gather(_bf16_dev(x), _to_dev(idx))
    rows = np.unique(np.concatenate([np.arange(16), np.arange(T * k - 16, T * k), rng.choice(T * k, 96, replace=False)]))
    ref = orc.quantize_mxfp8_rowwise(x[idx[rows]])
    assert np.array_equal(_np(codes)[rows], ref[0])
    assert np.array_equal(_np(scale)[:, rows], ref[1])

