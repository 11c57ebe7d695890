"""Benchmark of the block-scaled MoE expert grouped GEMM path on one MI355X.

One step = the whole hot path over one batch of the 32-expert shard
(hidden 7168, intermediate 2048, 32768 routed token-slots, Zipf(1.1) expert
popularity), inputs resident in HBM:
  forward  : NVFP4-variant quantize of W_gu, W_down (once per weight version,
             i.e. every optimizer step) and of X; gate/up grouped GEMM with
             the SwiGLU harness activation in its epilogue (writes H only);
             NVFP4-variant quantize of H; down grouped GEMM;
  backward : MXFP8 quantize of dY (row-wise and per-expert transposed), of the
             weights (transposed) and of H, dGU, X (transposed); dgrad and
             wgrad grouped GEMMs of the down and the gate/up projections.
dGU is synthetic N(0, 1e-3) (the backward workload's own input).

Prints ONE JSON line: metric/value = grouped-GEMM TFLOP/s of the whole step
(all six GEMMs' algorithmic flops / step time), per-stage breakdown (HIP-event
times on the stream the kernels run on), the roofline of the dominant kernel
and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --mode copy      # plain device copy (counter calibration)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"f16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}  # dense MFMA TFLOP/s (MI355X)
HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["step", "copy"], default="step")
    return ap.parse_args()


def copy_mode():
    """1 GiB device-to-device copy, three launches: the calibration kernel for
    the FETCH_SIZE / WRITE_SIZE counters, and the practical HBM ceiling of a
    read-write stream (timed with HIP events)."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    a.record()
    for _ in range(3):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 3
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "launches": 4,
                      "ms_per_copy": round(ms, 4), "gbps": round(2 * n / (ms * 1e-3) / 1e9, 1)}))


def build_step(bsq, torch, dev, cfg, counts, seed):
    """Device inputs, preallocated outputs and the stage list of one step of
    the expert shard ``cfg`` (routed token counts ``counts``): the forward of
    the NVFP4-variant path and the MXFP8 backward of both projections.  The
    step allocates nothing."""
    import numpy as np
    from workloads import offsets_from_counts

    E, Hd, I, M = cfg.n_experts, cfg.hidden, cfg.inter, cfg.m_total
    off_np = offsets_from_counts(counts)
    gen = torch.Generator(device=dev).manual_seed(seed)
    bf = torch.bfloat16

    def randn(shape, sigma=1.0):
        return (torch.randn(shape, generator=gen, device=dev) * sigma).to(bf)

    t = {}
    t["x"] = randn((M, Hd))
    t["w_gu"] = randn((E * 2 * I, Hd), 0.02)       # [E][2I][H]: gate rows then up rows
    t["w_dn"] = randn((E * Hd, I), 0.02)           # [E][H][I]
    t["dy"] = randn((M, Hd), 1e-3)
    t["dgu"] = randn((M, 2 * I), 1e-3)
    off = torch.from_numpy(off_np).to(dev)
    t["off"] = off
    woff_gu = torch.arange(E + 1, dtype=torch.int32, device=dev) * (2 * I)
    woff_dn = torch.arange(E + 1, dtype=torch.int32, device=dev) * Hd
    t["ws_f"] = ws_f = torch.empty(bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_FWD, E, M, 8192, 8192), dtype=torch.uint8,
                                   device=dev)
    t["ws_b"] = ws_b = torch.empty(bsq.bsq_workspace_size(bsq.BSQ_OP_GEMM_BWD, E, M, 8192, 8192), dtype=torch.uint8,
                                   device=dev)

    def nv(rows, cols):
        return (torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
                torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
                torch.empty((rows,), dtype=torch.float32, device=dev))

    def mxr(rows, cols):
        return (torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                torch.empty((cols // 32, rows), dtype=torch.uint8, device=dev))  # block-major scales

    def mxc(rows, cols, groups):
        P = bsq.bsq_colwise_padded_cols(groups, rows)
        return (torch.empty((cols, P), dtype=torch.uint8, device=dev),
                torch.empty((P // 32, cols), dtype=torch.uint8, device=dev))  # block-major scales

    x, w_gu, w_dn, dy, dgu = t["x"], t["w_gu"], t["w_dn"], t["dy"], t["dgu"]
    t["q_wgu"], t["q_wdn"], t["q_x"], t["q_h"] = q_wgu, q_wdn, q_x, q_h = (nv(E * 2 * I, Hd), nv(E * Hd, I), nv(M, Hd),
                                                                          nv(M, I))
    t["gu"] = gu = torch.empty((M, 2 * I), dtype=bf, device=dev)
    t["h"] = h = torch.empty((M, I), dtype=bf, device=dev)
    y = torch.empty((M, Hd), dtype=bf, device=dev)
    q_dy, q_dgu = mxr(M, Hd), mxr(M, 2 * I)
    t_wdn, t_wgu = mxc(E * Hd, I, E), mxc(E * 2 * I, Hd, E)
    t_dy, t_h, t_dgu, t_x = mxc(M, Hd, E), mxc(M, I, E), mxc(M, 2 * I, E), mxc(M, Hd, E)
    dh = torch.empty((M, I), dtype=bf, device=dev)
    dx = torch.empty((M, Hd), dtype=bf, device=dev)
    dw_dn = torch.empty((E, Hd, I), dtype=bf, device=dev)
    dw_gu = torch.empty((E, 2 * I, Hd), dtype=bf, device=dev)
    t["keep"] = (y, q_dy, q_dgu, t_wdn, t_wgu, t_dy, t_h, t_dgu, t_x, dh, dx, dw_dn, dw_gu)

    C = bsq.BSQ_COLWISE_T
    stages = [
        ("quant_nvfp4v_weights", lambda: (bsq.bsq_quantize_nvfp4v(w_gu, *q_wgu), bsq.bsq_quantize_nvfp4v(w_dn, *q_wdn))),
        ("quant_nvfp4v_x", lambda: bsq.bsq_quantize_nvfp4v(x, *q_x)),
        # gate/up GEMM with the harness activation H = silu(gate) * up in its
        # epilogue: the gate/up output never reaches HBM
        ("gemm_fwd_gate_up", lambda: bsq.bsq_grouped_gemm_fwd_swiglu(q_x, q_wgu, off, I, Hd, h=h, workspace=ws_f)),
        ("quant_nvfp4v_h", lambda: bsq.bsq_quantize_nvfp4v(h, *q_h)),
        ("gemm_fwd_down", lambda: bsq.bsq_grouped_gemm_fwd(q_h, q_wdn, off, Hd, I, y=y, workspace=ws_f)),
        # dY and dGU feed dgrad row-wise and wgrad per expert column: both layouts from one read
        ("quant_mxfp8_dual", lambda: (bsq.bsq_quantize_mxfp8_dual(dy, off, row=q_dy, t=t_dy),
                                      bsq.bsq_quantize_mxfp8_dual(dgu, off, row=q_dgu, t=t_dgu))),
        ("quant_mxfp8_colwise_t", lambda: (
            bsq.bsq_quantize_mxfp8(w_dn, C, offsets=woff_dn, codes=t_wdn[0], scale=t_wdn[1]),
            bsq.bsq_quantize_mxfp8(w_gu, C, offsets=woff_gu, codes=t_wgu[0], scale=t_wgu[1]),
            bsq.bsq_quantize_mxfp8(h, C, offsets=off, codes=t_h[0], scale=t_h[1]),
            bsq.bsq_quantize_mxfp8(x, C, offsets=off, codes=t_x[0], scale=t_x[1]))),
        ("gemm_bwd_dgrad_down", lambda: bsq.bsq_grouped_gemm_bwd(off, M, Hd, I, dy_q=q_dy, wt_q=t_wdn,
                                                                 flags=bsq.BSQ_DGRAD, dx=dh, workspace=ws_b)),
        ("gemm_bwd_wgrad_down", lambda: bsq.bsq_grouped_gemm_bwd(off, M, Hd, I, dyt_q=t_dy, xt_q=t_h,
                                                                 flags=bsq.BSQ_WGRAD, dw=dw_dn, workspace=ws_b)),
        ("gemm_bwd_dgrad_gate_up", lambda: bsq.bsq_grouped_gemm_bwd(off, M, 2 * I, Hd, dy_q=q_dgu, wt_q=t_wgu,
                                                                    flags=bsq.BSQ_DGRAD, dx=dx, workspace=ws_b)),
        ("gemm_bwd_wgrad_gate_up", lambda: bsq.bsq_grouped_gemm_bwd(off, M, 2 * I, Hd, dyt_q=t_dgu, xt_q=t_x,
                                                                    flags=bsq.BSQ_WGRAD, dw=dw_gu, workspace=ws_b)),
    ]
    flops = {
        "gemm_fwd_gate_up": 2.0 * M * 2 * I * Hd, "gemm_fwd_down": 2.0 * M * Hd * I,
        "gemm_bwd_dgrad_down": 2.0 * M * Hd * I, "gemm_bwd_wgrad_down": 2.0 * M * Hd * I,
        "gemm_bwd_dgrad_gate_up": 2.0 * M * 2 * I * Hd, "gemm_bwd_wgrad_gate_up": 2.0 * M * 2 * I * Hd,
    }
    nvb = lambda r, c: 2 * r * c + r * c // 2 + r * c // 16 + 4 * r           # bf16 in + codes + scales + rscale
    mxb = lambda r, c: 2 * r * c + r * c + r * c // 32                       # bf16 in + codes + scales
    mxd = lambda r, c: 2 * r * c + 2 * (r * c + r * c // 32)                 # one read, two layouts out
    qbytes = {
        "quant_nvfp4v_weights": nvb(E * 2 * I, Hd) + nvb(E * Hd, I), "quant_nvfp4v_x": nvb(M, Hd),
        "quant_nvfp4v_h": nvb(M, I), "quant_mxfp8_dual": mxd(M, Hd) + mxd(M, 2 * I),
        "quant_mxfp8_colwise_t": mxb(E * Hd, I) + mxb(E * 2 * I, Hd) + mxb(M, I) + mxb(M, Hd),
    }
    return t, stages, flops, qbytes


def time_step(torch, stages, steps, warmup):
    """Wall time per step over exactly ``steps`` steps (nothing else in the
    timed region), then a second, instrumented pass with HIP events around
    every stage on the launch stream.  Returns (ms per step, ms per step of
    the instrumented pass, median ms per stage)."""
    import numpy as np
    stream = torch.cuda.current_stream()

    def step(events=None):
        for i, (_, fn) in enumerate(stages):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in stages]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(steps):
        step(ev[s])
    torch.cuda.synchronize()
    ms_instr = (time.perf_counter() - t1) * 1e3 / steps
    stage_ms = {nm: float(np.median([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]))
                for i, (nm, _) in enumerate(stages)}
    return ms_step, ms_instr, stage_ms


def breakdown_of(stage_ms, flops, qbytes):
    out = {}
    for nm, ms in stage_ms.items():
        d = {"ms": round(ms, 4)}
        if nm in flops:
            tf = flops[nm] / (ms * 1e-3) / 1e12
            peak = PEAK["f16"] if "fwd" in nm else PEAK["fp8"]
            d.update({"tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / peak, 4),
                      "mfma": "f16 (exact E2M1xE4M3 dequant)" if "fwd" in nm else "fp8 e4m3 block-scaled"})
        if nm in qbytes:
            gbs = qbytes[nm] / (ms * 1e-3) / 1e9
            d.update({"gbps": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_GBS, 4)})
        out[nm] = d
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is built and measured "
              f"for a single MI355X", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        copy_mode()
        return
    import numpy as np
    import torch

    if not os.path.exists(os.path.join(ROOT, "block_scaled_precision_bsq_amd", "libbsq.so")):
        from __graft_entry__ import build
        build()
    import block_scaled_precision_bsq_amd as bsq
    from workloads import CONFIGS, moe_counts, offsets_from_counts

    cfg = CONFIGS[3]
    E, Hd, I, M = cfg.n_experts, cfg.hidden, cfg.inter, cfg.m_total
    counts = moe_counts(cfg)
    off_np = offsets_from_counts(counts)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t, stages, flops, qbytes = build_step(bsq, torch, dev, cfg, counts, 20250)
    ms_step, ms_step_instr, stage_ms = time_step(torch, stages, args.steps, args.warmup)
    total_flops = sum(flops.values())
    breakdown = breakdown_of(stage_ms, flops, qbytes)
    dom = max(flops, key=lambda k: stage_ms[k])
    dom_tf = flops[dom] / (stage_ms[dom] * 1e-3) / 1e12
    dom_peak = PEAK["f16"] if "fwd" in dom else PEAK["fp8"]
    traffic = measured_traffic()
    for nm, b in traffic.items():
        if nm in breakdown:
            breakdown[nm]["hbm_bytes_measured"] = b
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(dom_tf, 1), "peak": dom_peak,
                "unit": "TFLOP/s", "frac": round(dom_tf / dom_peak, 4), "traffic": traffic.get(dom)}

    quant = quantize_config2(bsq, torch, dev)
    x, w_gu, w_dn, h, off, ws_f = t["x"], t["w_gu"], t["w_dn"], t["h"], t["off"], t["ws_f"]
    unfused = unfused_gate_up(bsq, torch, t, off, I, Hd, stage_ms)
    plain_ms = {"gemm_fwd_gate_up": unfused["gemm_fwd_gate_up_plain_ms"], "gemm_fwd_down": stage_ms["gemm_fwd_down"]}
    fwd_mx = fwd_mxfp8_compare(bsq, torch, dev, x, w_gu, w_dn, h, off, E, Hd, I, M, plain_ms, ws_f)
    bf16_base = bf16_baseline(bsq, torch, dev, x, w_gu, w_dn, h, off, E, Hd, I, M, plain_ms, fwd_mx, ws_f)
    frozen = frozen_w4a16(bsq, torch, dev, x, h, t["q_wgu"], t["q_wdn"], off, E, Hd, I, M, bf16_base, ws_f)
    del t, stages, x, w_gu, w_dn, h, off, ws_f
    torch.cuda.empty_cache()
    cfg5 = config5_line(bsq, torch, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, counts, off_np)
    value = total_flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "grouped-GEMM TFLOP/s (% of MFMA peak) + quantize GB/s, 32 experts 7168x2048",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fwd: E2M1xE4M3 dequantized exactly to f16, f16 MFMA; bwd: E4M3 block-scaled MFMA; fp32 accumulate",
        "data": "synthetic (seeded torch.randn; Zipf(1.1) expert counts)",
        "config": {"workload": "MoE expert shard fwd+bwd: 32 experts, hidden 7168, intermediate 2048, "
                               "32768 routed token-slots, Zipf(1.1); NVFP4-variant fwd, MXFP8 bwd",
                   "experts": E, "hidden": Hd, "intermediate": I, "token_slots": M,
                   "gemm_tflop_per_step": round(total_flops / 1e12, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "stage_times": "median over the K steps of HIP events around each stage on the launch stream",
        "ms_per_step_instrumented": round(ms_step_instr, 4),
        "quantize": quant,
        "config5": cfg5,
        "gate_up_unfused": unfused,
        "fwd_mxfp8": fwd_mx,
        "bf16_baseline": bf16_base,
        "frozen_w4a16": frozen,
    }
    print(json.dumps(out))


def unfused_gate_up(bsq, torch, t, off, I, Hd, stage_ms, reps=10):
    """The gate/up projection without the fused epilogue, on the same tensors
    outside the step: the plain NVFP4v GEMM writing gu (bf16 [gate | up]),
    then the SwiGLU + NVFP4v quantize kernel reading it back.  Median of
    per-launch HIP events; compared with the step's fused GEMM + quantize of H."""
    stream = torch.cuda.current_stream()
    q_x, q_wgu, gu, h, q_h, ws_f = t["q_x"], t["q_wgu"], t["gu"], t["h"], t["q_h"], t["ws_f"]

    def med(fn):
        for _ in range(2):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return ts[len(ts) // 2]

    g = med(lambda: bsq.bsq_grouped_gemm_fwd(q_x, q_wgu, off, 2 * I, Hd, y=gu, workspace=ws_f))
    sq = med(lambda: bsq.bsq_swiglu_quantize_nvfp4v(gu, h=h, codes=q_h[0], bscale=q_h[1], rscale=q_h[2]))
    fused = stage_ms["gemm_fwd_gate_up"] + stage_ms["quant_nvfp4v_h"]
    return {"gemm_fwd_gate_up_plain_ms": round(g, 4), "swiglu_quant_nvfp4v_ms": round(sq, 4),
            "unfused_total_ms": round(g + sq, 4), "fused_total_ms": round(fused, 4),
            "note": "fused = gate/up GEMM with SwiGLU in its epilogue writing H, then the NVFP4v quantize of H "
                    "(the step's two stages); unfused = GEMM writing gu, then SwiGLU fused with H's quantize"}


def config5_line(bsq, torch, dev, steps=10, warmup=3):
    """The large, imbalanced shard: 48 experts (one GPU's share of a
    384-expert MoE), 8 of them empty, Zipf(1.5) over the other 40, 65536
    token-slots, hidden 7168, intermediate 2048; the same step as the
    headline workload (every quantization and the six grouped GEMMs)."""
    from workloads import CONFIGS, moe_counts
    cfg = CONFIGS[5]
    counts = moe_counts(cfg)
    t, stages, flops, qbytes = build_step(bsq, torch, dev, cfg, counts, 50505)
    ms_step, _, stage_ms = time_step(torch, stages, steps, warmup)
    fwd = sum(v for k, v in flops.items() if "fwd" in k)
    bwd = sum(v for k, v in flops.items() if "bwd" in k)
    fwd_ms = sum(stage_ms[k] for k in flops if "fwd" in k)
    bwd_ms = sum(stage_ms[k] for k in flops if "bwd" in k)
    out = {"workload": "48 experts (8 empty), Zipf(1.5) over 40, 65536 token-slots, hidden 7168, intermediate 2048",
           "max_tokens_per_expert": int(max(counts)), "min_nonempty": int(min(c for c in counts if c > 0)),
           "steps": steps, "ms_per_step": round(ms_step, 4),
           "gemm_tflops_per_step": round(sum(flops.values()) / (ms_step * 1e-3) / 1e12, 1),
           "fwd_gemm_tflop": round(fwd / 1e12, 3), "fwd_gemm_ms": round(fwd_ms, 4),
           "fwd_gemm_tflops": round(fwd / (fwd_ms * 1e-3) / 1e12, 1),
           "bwd_gemm_tflop": round(bwd / 1e12, 3), "bwd_gemm_ms": round(bwd_ms, 4),
           "bwd_gemm_tflops": round(bwd / (bwd_ms * 1e-3) / 1e12, 1),
           "breakdown": breakdown_of(stage_ms, flops, qbytes)}
    del t, stages
    torch.cuda.empty_cache()
    return out


def quantize_config2(bsq, torch, dev, reps=20):
    """Quantize-only workload: 16384 tokens x 7168 hidden bf16 ~N(0,1) with
    1% (72) outlier channels scaled x50.  Algorithmic bytes: bf16 read plus
    codes and scales written; HIP events on the launch stream."""
    R, C = 16384, 7168
    gen = torch.Generator(device=dev).manual_seed(2002)
    x = torch.randn((R, C), generator=gen, device=dev)
    cols = torch.randperm(C, generator=gen, device=dev)[:72]
    x[:, cols] *= 50.0
    x = x.to(torch.bfloat16)
    one = torch.tensor([0, R], dtype=torch.int32, device=dev)
    nv = (torch.empty((R, C // 2), dtype=torch.uint8, device=dev), torch.empty((R, C // 16), dtype=torch.uint8, device=dev),
          torch.empty((R,), dtype=torch.float32, device=dev))
    mr = (torch.empty((R, C), dtype=torch.uint8, device=dev), torch.empty((C // 32, R), dtype=torch.uint8, device=dev))
    P = bsq.bsq_colwise_padded_cols(1, R)
    mc = (torch.empty((C, P), dtype=torch.uint8, device=dev), torch.empty((P // 32, C), dtype=torch.uint8, device=dev))
    cases = {
        "nvfp4v": (lambda: bsq.bsq_quantize_nvfp4v(x, *nv), 2 * R * C + R * C // 2 + R * C // 16 + 4 * R),
        "mxfp8_rowwise": (lambda: bsq.bsq_quantize_mxfp8(x, bsq.BSQ_ROWWISE, codes=mr[0], scale=mr[1]),
                          2 * R * C + R * C + R * C // 32),
        "mxfp8_colwise_t": (lambda: bsq.bsq_quantize_mxfp8(x, bsq.BSQ_COLWISE_T, offsets=one, codes=mc[0], scale=mc[1]),
                            2 * R * C + C * P + C * P // 32),
        # both layouts from one read (against the two calls above: one bf16 read saved)
        "mxfp8_dual": (lambda: bsq.bsq_quantize_mxfp8_dual(x, one, row=mr, t=mc),
                       2 * R * C + R * C + R * C // 32 + C * P + C * P // 32),
    }
    stream = torch.cuda.current_stream()
    # 512 MB read before every timed launch: more than the 256 MB Infinity
    # Cache, so no launch finds its input (235 MB) cached by the previous one;
    # a read leaves clean lines, so the launch pays no write-back of the
    # eviction pass (the previous launch's outputs are written back during it)
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    out = {"workload": "quantize: 16384 x 7168 bf16 N(0,1), 72 outlier channels x50",
           "timing": f"median of {reps} launches, each after a 512 MB read that evicts the 256 MB Infinity Cache; "
                     "HIP events on the launch stream around the launch alone"}

    def timed(fn):
        for _ in range(3):
            fn()
        ts = []
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            flush.amax()
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        return ts[len(ts) // 2]

    for name, (fn, nbytes) in cases.items():
        us = timed(fn)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "bytes": nbytes, "gbps": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_GBS, 4)}
    # Dispatch-style quantize: 4096 tokens of the same data, top-8 routing into
    # 32768 expert-sorted slots, permutation fused into the MXFP8 quantizer.
    T, k = 4096, 8
    picks = torch.argsort(torch.rand((T, 32), generator=gen, device=dev), dim=1)[:, :k]
    idx = (torch.argsort(picks.reshape(-1), stable=True) // k).to(torch.int32)
    gc = torch.empty((T * k, C), dtype=torch.uint8, device=dev)
    gs = torch.empty((C // 32, T * k), dtype=torch.uint8, device=dev)
    xs = x[:T]
    us = timed(lambda: bsq.bsq_quantize_mxfp8_gather(xs, idx, codes=gc, scale=gs))
    nbytes = 2 * T * k * C + T * k * C + T * k * C // 32   # gathered bf16 rows read + codes + scales
    nmin = 2 * T * C + T * k * C + T * k * C // 32         # each source row once + codes + scales
    out["mxfp8_gather_dispatch"] = {"workload": "4096 tokens x 7168, top-8 into 32768 expert-sorted slots",
                                    "us": round(us, 2), "bytes_gathered": nbytes,
                                    "gbps_gathered": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes_min": nmin,
                                    "gbps_min": round(nmin / (us * 1e-6) / 1e9, 1)}
    # Ablation (not the method): the same quantizer with fast approximate
    # divides; how many decisions it changes against IEEE division, and its time.
    bsq.bsq_quantize_nvfp4v(x, *nv)
    fc, fb, fr = bsq.bsq_debug_quantize_nvfp4v_fastdiv(x)
    us = timed(lambda: bsq.bsq_debug_quantize_nvfp4v_fastdiv(x))
    nib = lambda c: torch.stack([c & 15, c >> 4], -1)
    out["nvfp4v_fastdiv_ablation"] = {
        "us": round(us, 2), "speedup_vs_ieee": round(out["nvfp4v"]["us"] / us, 3),
        "codes_changed_frac": float((nib(fc) != nib(nv[0])).double().mean()),
        "bscale_changed_frac": float((fb != nv[1]).double().mean()),
        "rscale_changed_frac": float((fr != nv[2]).double().mean()),
    }
    return out


def fwd_mxfp8_compare(bsq, torch, dev, x, w_gu, w_dn, h, off, E, Hd, I, M, nv_ms, ws, reps=10):
    """The forward expert GEMMs again with all-MXFP8 operands (ROWWISE X, H and
    weights; block-scaled fp8 MFMA) on the same tensors, outside the step:
    the MXFP8 alternative to the NVFP4-variant forward.  HIP events on the
    launch stream; quantization not timed."""
    R = bsq.BSQ_ROWWISE
    q = {"x": bsq.bsq_quantize_mxfp8(x, R), "w_gu": bsq.bsq_quantize_mxfp8(w_gu, R),
         "h": bsq.bsq_quantize_mxfp8(h, R), "w_dn": bsq.bsq_quantize_mxfp8(w_dn, R)}
    y_gu = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((M, Hd), dtype=torch.bfloat16, device=dev)
    cases = {
        "gemm_fwd_gate_up": (lambda: bsq.bsq_grouped_gemm_fwd_mxfp8(q["x"], q["w_gu"], off, 2 * I, Hd, y=y_gu,
                                                                    workspace=ws), 2.0 * M * 2 * I * Hd),
        "gemm_fwd_down": (lambda: bsq.bsq_grouped_gemm_fwd_mxfp8(q["h"], q["w_dn"], off, Hd, I, y=y_dn,
                                                                 workspace=ws), 2.0 * M * Hd * I),
    }
    stream = torch.cuda.current_stream()
    out = {"operands": "MXFP8 ROWWISE activations and weights, block-scaled fp8 MFMA, bf16 out"}
    for name, (fn, fl) in cases.items():
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / PEAK["fp8"], 4),
                     "speedup_vs_nvfp4v_fwd": round(nv_ms[name] / ms, 3)}
    del q, y_gu, y_dn
    return out


def bf16_baseline(bsq, torch, dev, x, w_gu, w_dn, h, off, E, Hd, I, M, stage_ms, fwd_mx, ws, reps=10):
    """The forward expert GEMMs on plain bf16 operands with the same tiles,
    pipeline and scheduler (bsq_grouped_gemm_bf16), outside the step: the
    baseline the block-scaled GEMMs are compared with."""
    y_gu = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((M, Hd), dtype=torch.bfloat16, device=dev)
    cases = {
        "gemm_fwd_gate_up": (lambda: bsq.bsq_grouped_gemm_bf16(x, w_gu, off, 2 * I, Hd, y=y_gu, workspace=ws),
                             2.0 * M * 2 * I * Hd),
        "gemm_fwd_down": (lambda: bsq.bsq_grouped_gemm_bf16(h, w_dn, off, Hd, I, y=y_dn, workspace=ws),
                          2.0 * M * Hd * I),
    }
    stream = torch.cuda.current_stream()
    out = {"operands": "bf16 activations and weights, bf16 MFMA, bf16 out"}
    for name, (fn, fl) in cases.items():
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / PEAK["f16"], 4),
                     "speedup_nvfp4v_fwd_vs_bf16": round(ms / stage_ms[name], 3),
                     "speedup_mxfp8_fwd_vs_bf16": round(ms / fwd_mx[name]["ms"], 3)}
    del y_gu, y_dn
    return out


def frozen_w4a16(bsq, torch, dev, x, h, q_wgu, q_wdn, off, E, Hd, I, M, bf16_base, ws, reps=10):
    """Frozen experts in packed storage: the forward expert GEMMs with bf16
    activations against the NVFP4-variant weights of the step (4.5 bits per
    weight), dequantized to bf16 inside the kernel (bsq_grouped_gemm_w4a16),
    outside the step; compared with the bf16 baseline on the same shapes."""
    y_gu = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((M, Hd), dtype=torch.bfloat16, device=dev)
    wbytes = lambda q: sum(t.numel() * t.element_size() for t in q)
    cases = {
        "gemm_fwd_gate_up": (lambda: bsq.bsq_grouped_gemm_w4a16(x, q_wgu, off, 2 * I, Hd, y=y_gu, workspace=ws),
                             2.0 * M * 2 * I * Hd, wbytes(q_wgu), 2 * E * 2 * I * Hd),
        "gemm_fwd_down": (lambda: bsq.bsq_grouped_gemm_w4a16(h, q_wdn, off, Hd, I, y=y_dn, workspace=ws),
                          2.0 * M * Hd * I, wbytes(q_wdn), 2 * E * Hd * I),
    }
    stream = torch.cuda.current_stream()
    out = {"operands": "bf16 activations, NVFP4-variant packed weights dequantized to bf16 in-kernel, bf16 MFMA"}
    for name, (fn, fl, wb, wb16) in cases.items():
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / PEAK["f16"], 4),
                     "weight_bytes": wb, "weight_bytes_bf16": wb16, "weight_compression": round(wb16 / wb, 3),
                     "speedup_vs_bf16": round(bf16_base[name]["ms"] / ms, 3)}
    del y_gu, y_dn
    return out


def kernel_source_hash(stage):
    """Hash of the code a stage's kernel is built from (kernel file plus the
    shared headers, comments and blank space removed), used to tell whether
    stored counter readings still describe the kernel as it is now."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "block_scaled_precision_bsq_amd", "csrc")
    main = ("gemm_fwd.hip" if stage.startswith("gemm_fwd") else "gemm_bwd.hip" if stage.startswith("gemm_bwd")
            else "quantize.hip")
    h = hashlib.sha256()
    for f in (main, "device_common.h", "gemm_common.h", "gemm_pipe.h"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)   # block comments
        code = re.sub(r"//[^\n]*", " ", code)                 # line comments
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    stored under profiles/ (scaled by the copy-kernel calibration); a stage
    whose kernel source changed since the counters were taken is left out."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_moe32_h7168_i2048.json")
    if not os.path.exists(path):
        return {}
    with open(path) as fh:
        table = json.load(fh)
    out = {}
    for stage, rec in table.get("stages", {}).items():
        if rec.get("source") == kernel_source_hash(stage):
            out[stage] = rec["bytes"]
    # multi-launch stages: sum of their launches when all are current
    for stage in ("quant_nvfp4v_weights", "quant_mxfp8_dual", "quant_mxfp8_colwise_t"):
        parts = [k for k in table.get("stages", {}) if k.startswith(stage + ":")]
        if parts and all(k in out for k in parts):
            out[stage] = sum(out[k] for k in parts)
    return out


def host_cpu():
    """CPU model and core counts of the host, read at run time."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": usable, "os_cpu_count": os.cpu_count()}


def cpu_quantize_rates(oracle, threads):
    """The oracle's quantizers on a bounded sample of the quantize-only
    workload (rows of 7168 bf16 ~N(0,1) with 72 outlier channels x50):
    algorithmic GB/s on ``threads`` threads and on one thread."""
    from workloads import make_quantize_input, rng_for
    C = 7168
    x = make_quantize_input(rng_for(2, salt=91), 2048, C)
    cases = {"nvfp4v": (oracle.quantize_nvfp4v, lambda r: 2 * r * C + r * C // 2 + r * C // 16 + 4 * r),
             "mxfp8_rowwise": (oracle.quantize_mxfp8_rowwise, lambda r: 2 * r * C + r * C + r * C // 32)}
    out = {"sample": f"2048 x {C} rows (all threads) and 256 x {C} rows (one thread) of the 16384 x {C} "
                     "quantize-only workload; best of 3"}
    for name, (fn, nbytes) in cases.items():
        d = {}
        for nthr, rows in ((threads, 2048), (1, 256)):
            oracle.set_num_threads(nthr)
            xs = x[:rows]
            best = float("inf")
            for _ in range(3):
                t0 = time.perf_counter()
                fn(xs)
                best = min(best, time.perf_counter() - t0)
            d["gbps_all_threads" if nthr == threads else "gbps_one_thread"] = round(nbytes(rows) / best / 1e9, 4)
        d["threads"] = threads
        out[name] = d
    oracle.set_num_threads(threads)
    return out


def cpu_baseline(cfg, counts, off_np):
    """The oracle as it stands, on a bounded sample of the same step: for one
    expert at a time, largest first, every quantization and all six GEMMs of
    the step (forward gate/up, SwiGLU, forward down, dgrad and wgrad of both
    projections) on that expert's rows, until about ``budget_s`` seconds of
    oracle time are spent.  Rate = the GEMM flops of the experts done / the
    oracle time (quantization included, input generation not).  Also the
    oracle's quantizers alone, on all threads and on one."""
    import numpy as np

    import oracle
    from workloads import normal_bf16, rng_for
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = os.cpu_count() or 1
    host = host_cpu()
    omp_threads = oracle.max_threads()
    rng = rng_for(3, salt=55)
    Hd, I = cfg.hidden, cfg.inter
    budget_s = 20.0  # the sample stops after the first expert that ends past this
    flops = 0.0
    done = []
    t_all = 0.0
    for e in [int(e) for e in np.argsort(-np.asarray(counts), kind="stable")]:
        m = int(counts[e])
        if m == 0:
            break
        x, dy = normal_bf16(rng, (m, Hd)), normal_bf16(rng, (m, Hd), 1e-3)
        dgu = normal_bf16(rng, (m, 2 * I), 1e-3)
        w_gu, w_d = normal_bf16(rng, (2 * I, Hd), 0.02), normal_bf16(rng, (Hd, I), 0.02)
        seg = np.array([0, m], np.int32)
        t0 = time.perf_counter()
        # forward: NVFP4-variant operands
        gu = oracle.grouped_gemm_fwd(oracle.quantize_nvfp4v(x), oracle.quantize_nvfp4v(w_gu), seg)
        h = oracle.round_bf16(oracle.swiglu(gu))
        oracle.grouped_gemm_fwd(oracle.quantize_nvfp4v(h), oracle.quantize_nvfp4v(w_d), seg)
        # backward of the down projection: MXFP8 operands
        oracle.grouped_gemm_dgrad(oracle.quantize_mxfp8_rowwise(dy),
                                  oracle.quantize_mxfp8_colwise_t(w_d, np.array([0, Hd], np.int32)), seg, Hd)
        oracle.grouped_gemm_wgrad(oracle.quantize_mxfp8_colwise_t(dy, seg),
                                  oracle.quantize_mxfp8_colwise_t(h, seg), seg)
        # backward of the gate/up projection
        oracle.grouped_gemm_dgrad(oracle.quantize_mxfp8_rowwise(dgu),
                                  oracle.quantize_mxfp8_colwise_t(w_gu, np.array([0, 2 * I], np.int32)), seg, 2 * I)
        oracle.grouped_gemm_wgrad(oracle.quantize_mxfp8_colwise_t(dgu, seg),
                                  oracle.quantize_mxfp8_colwise_t(x, seg), seg)
        t_all += time.perf_counter() - t0
        flops += 3 * 2.0 * m * (2 * I * Hd + Hd * I)
        done.append(m)
        if t_all >= budget_s:
            break
    quant = cpu_quantize_rates(oracle, omp_threads)
    return {"value": round(flops / t_all / 1e12, 5), "unit": "TFLOP/s", "cores": int(max(blas_threads, omp_threads)),
            "kind": "oracle",
            "sample": f"the whole step (NVFP4-variant and MXFP8 quantizations, SwiGLU, float64 forward, dgrad and "
                      f"wgrad GEMMs of both projections) for the {len(done)} largest of {len(counts)} experts "
                      f"({sum(done)} of {int(np.sum(counts))} token-slots); stops after ~{budget_s:.0f} s; "
                      f"seconds={t_all:.1f}",
            "threads": {"blas_float64_gemm": int(blas_threads), "openmp_quantizers": int(omp_threads)},
            **host, "quantize": quant}


if __name__ == "__main__":
    main()
