"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and lays them out: it holds none of the
quantization or GEMM arithmetic, so both the CPU oracle and the HIP path can be
fed from it without sharing any of the method's code.

The shapes follow the workloads the pages name for the MoE expert GEMM
("Scaling and Optimizing Frontier Model Training (Fireworks AI)" summary, key
claim on MXFP8 expert kernels: 32 experts per rank, hidden 7168, intermediate
2048) and the 384-expert, top-8 MoE class of the same summary.  Readings of
distributions the pages leave open:

* ``N(mu, sigma)`` takes sigma as a standard deviation; ``lognormal(0,1)`` is
  ``exp(N(0,1))``.
* "1% outlier channels" is ``round(0.01 * cols)`` columns, picked by a seeded
  permutation and multiplied by 50.
* Zipf(s) popularity is ``P(rank r) ∝ r**-s``; counts come from largest
  remainder rounding of ``total * p``; ranks map to expert ids through a seeded
  permutation.  Empty experts (the 48-expert shard) sit at seeded positions.
* fp32 samples become bf16 by round-to-nearest-even, as ``torch.to`` does.

Every generator takes a ``numpy.random.Generator`` (PCG64) so callers control
the seed; ``rng_for(cfg)`` gives the canonical seed ``1000 + cfg``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "rng_for", "f32_to_bf16_bits", "bf16_bits_to_f32", "normal_bf16",
    "zipf_counts", "offsets_from_counts", "top2_uniform_routing", "Config",
    "CONFIGS", "make_quantize_input", "make_expert_weights",
]


def rng_for(cfg: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 + cfg + 7919 * salt))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Input preparation only (the method starts from bf16 tensors); NaN is not
    produced by the generators and is not handled.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u.astype(np.uint64) + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def zipf_counts(total: int, n: int, s: float) -> np.ndarray:
    """Counts per popularity rank (rank 1 first), summing to ``total``."""
    r = np.arange(1, n + 1, dtype=np.float64)
    p = r ** -s
    p /= p.sum()
    raw = total * p
    base = np.floor(raw).astype(np.int64)
    rem = int(total - base.sum())
    order = np.argsort(-(raw - base), kind="stable")
    base[order[:rem]] += 1
    return base


def offsets_from_counts(counts) -> np.ndarray:
    c = np.asarray(counts, dtype=np.int64)
    off = np.zeros(len(c) + 1, dtype=np.int32)
    off[1:] = np.cumsum(c)
    return off


def expert_counts_zipf(rng, total, n_experts, s, n_empty=0) -> np.ndarray:
    """Per-expert token counts: Zipf over the non-empty experts, ranks
    shuffled onto expert ids, ``n_empty`` experts at seeded positions."""
    live = n_experts - n_empty
    per_rank = zipf_counts(total, live, s)
    perm = rng.permutation(n_experts)
    empty = set(perm[:n_empty].tolist())
    live_ids = [e for e in perm[n_empty:].tolist()]
    counts = np.zeros(n_experts, dtype=np.int64)
    for rank, e in enumerate(live_ids):
        counts[e] = per_rank[rank]
    assert not any(counts[e] for e in empty)
    return counts


def top2_uniform_routing(rng, n_tokens, n_experts):
    """Each token picks two distinct experts uniformly.  Returns
    (slot_token, counts): the token index of each expert-sorted slot and the
    slot count per expert."""
    picks = np.stack([rng.choice(n_experts, size=2, replace=False) for _ in range(n_tokens)])
    slot_expert = picks.reshape(-1)
    slot_tok = np.repeat(np.arange(n_tokens), 2)
    order = np.argsort(slot_expert, kind="stable")
    counts = np.bincount(slot_expert, minlength=n_experts)
    return slot_tok[order], counts


def make_quantize_input(rng, rows, cols, outlier_frac=0.01, outlier_mult=50.0):
    """N(0,1) bf16 rows with ``round(outlier_frac*cols)`` outlier columns x50."""
    x = rng.standard_normal(size=(rows, cols), dtype=np.float32)
    n_out = int(round(outlier_frac * cols))
    if n_out:
        cols_out = rng.permutation(cols)[:n_out]
        x[:, cols_out] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def make_expert_weights(rng, n_experts, n, k, sigma=0.02):
    return normal_bf16(rng, (n_experts, n, k), sigma)


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    n_experts: int
    hidden: int
    inter: int
    m_total: int
    zipf_s: float | None
    n_empty: int = 0


CONFIGS = {
    1: Config(1, "tiny MoE FFN: 4 experts, hidden 256, intermediate 128, 512 tokens top-2", 4, 256, 128, 1024, None),
    2: Config(2, "quantize: 16384 x 7168 bf16 N(0,1), 1% outlier channels x50", 1, 7168, 0, 16384, None),
    3: Config(3, "32 experts, hidden 7168, intermediate 2048, 32768 slots, Zipf(1.1)", 32, 7168, 2048, 32768, 1.1),
    4: Config(4, "32 experts, hidden 7168, intermediate 2048, 32768 slots, Zipf(1.1), backward", 32, 7168, 2048, 32768, 1.1),
    5: Config(5, "48 experts (8 empty), hidden 7168, intermediate 2048, 65536 slots, Zipf(1.5)", 48, 7168, 2048, 65536, 1.5, 8),
}


def moe_counts(cfg: Config, rng=None) -> np.ndarray:
    """Expert token counts for configs 3-5 (configs 3 and 4 share them)."""
    if rng is None:
        rng = rng_for(3 if cfg.idx in (3, 4) else cfg.idx, salt=1)
    return expert_counts_zipf(rng, cfg.m_total, cfg.n_experts, cfg.zipf_s, cfg.n_empty)


def tiny_moe(seed_cfg: int = 1):
    """Config 1 inputs: token activations with per-token lognormal magnitude,
    top-2 uniform routing over 4 experts, N(0, 0.02) expert weights.
    Returns dict with expert-sorted activations ``x_sorted`` (bf16 bits),
    ``offsets``, ``w_gu`` [E][2*inter][hidden], ``w_down`` [E][hidden][inter]."""
    cfg = CONFIGS[1]
    rng = rng_for(seed_cfg)
    n_tok = 512
    mag = np.exp(rng.standard_normal(size=(n_tok, 1))).astype(np.float32)
    x = (rng.standard_normal(size=(n_tok, cfg.hidden), dtype=np.float32) * mag).astype(np.float32)
    x_bf = f32_to_bf16_bits(x)
    slot_tok, counts = top2_uniform_routing(rng, n_tok, cfg.n_experts)
    x_sorted = x_bf[slot_tok]
    w_gu = make_expert_weights(rng, cfg.n_experts, 2 * cfg.inter, cfg.hidden)
    w_down = make_expert_weights(rng, cfg.n_experts, cfg.hidden, cfg.inter)
    return dict(x_sorted=np.ascontiguousarray(x_sorted), offsets=offsets_from_counts(counts),
                w_gu=w_gu, w_down=w_down, slot_tok=slot_tok, counts=counts)
