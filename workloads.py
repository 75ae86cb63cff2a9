"""Seeded synthetic inputs for the block-scaled token codec.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the CPU oracle tests and the HIP path (tests, smoke run,
benchmark) take their inputs from here.

No page uses a public dataset; these generators stand in for the MoE token
rows, gradients and routings the pages describe.  Every tensor gets its own
child stream of ``numpy.random.SeedSequence(seed)`` in the order listed, and
float samples are rounded to BF16 by round-to-nearest-even on the bit pattern.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def to_bf16_bits(x):
    """float array -> BF16 bit patterns (uint16), round-to-nearest-even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)


def _streams(seed, n):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


@dataclass
class Workload:
    name: str
    x_bits: Optional[np.ndarray] = None          # [T, H] BF16 token rows / gradient rows
    topk_idx: Optional[np.ndarray] = None        # [T, k] int32 expert ids
    num_experts: int = 0
    alignment: int = 16
    sr_seed: Optional[int] = None
    sr_counter_base: int = 0
    preact_bits: Optional[np.ndarray] = None     # [T, 2F] BF16
    dy_bits: Optional[np.ndarray] = None         # [T, F] BF16
    counts: Optional[np.ndarray] = None          # [E] tokens per expert (expert-major rows)
    meta: dict = field(default_factory=dict)


def zipf_top2(rng, tokens, num_experts, alpha, empty):
    """Two distinct experts per token, Gumbel-top-2 on log p with p_e ~ (e+1)^-alpha, p_empty = 0."""
    p = (np.arange(num_experts) + 1.0) ** -alpha
    for e in empty:
        p[e] = 0.0
    p /= p.sum()
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    g = rng.gumbel(size=(tokens, num_experts)) + logp[None, :]
    return np.argsort(-g, axis=1, kind="stable")[:, :2].astype(np.int32)


def random_topk(rng, tokens, num_experts, k):
    """k distinct experts per token, uniform: top-k of standard normal logits (ties -> lower id)."""
    logits = rng.standard_normal((tokens, num_experts))
    return np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)


def config1(seed=0):
    """256 tokens x hidden 1024, N(0,1) with 0.1% outliers scaled x50; top-1 of 4 experts."""
    r = _streams(seed, 3)
    x = r[0].standard_normal((256, 1024))
    mask = r[1].random((256, 1024)) < 1e-3
    x[mask] *= 50.0
    topk = r[2].integers(0, 4, size=(256, 1)).astype(np.int32)
    return Workload("nvfp4-roundtrip-256x1024-e4-top1", x_bits=to_bf16_bits(x), topk_idx=topk,
                    num_experts=4, alignment=16)


def config2(seed=0):
    """4096 x 4096, N(0,1); top-2 of 8 experts, Zipf(1.2)-skewed, expert 7 empty; 16-row aligned."""
    r = _streams(seed, 2)
    x = r[0].standard_normal((4096, 4096))
    topk = zipf_top2(r[1], 4096, 8, 1.2, empty=[7])
    return Workload("dispatch-4096x4096-e8-top2-zipf1.2", x_bits=to_bf16_bits(x), topk_idx=topk,
                    num_experts=8, alignment=16)


def config3(seed=0):
    """DeepSeek-V3-shaped one-GPU share: 16384 x 7168, N(0, 0.5^2) * 10^U(-2,2) per token;
    top-8 of 32 experts from N(0,1) logits."""
    r = _streams(seed, 3)
    mag = 10.0 ** r[1].uniform(-2.0, 2.0, size=(16384, 1))
    x = r[0].standard_normal((16384, 7168), dtype=np.float32) * np.float32(0.5) * mag.astype(np.float32)
    topk = random_topk(r[2], 16384, 32, 8)
    return Workload("dsv3-share-16384x7168-e32-top8", x_bits=to_bf16_bits(x), topk_idx=topk,
                    num_experts=32, alignment=16)


def config4(seed=0):
    """Combine-backward gradients: 32768 x 4096, Student-t(3) * 1e-3; uniform 2-of-16 routing;
    stochastic rounding with seed 1234, counter base 0."""
    r = _streams(seed, 2)
    g = r[0].standard_t(3, size=(32768, 4096)) * 1e-3
    topk = random_topk(r[1], 32768, 16, 2)
    return Workload("combine-bwd-sr-32768x4096-e16-top2", x_bits=to_bf16_bits(g), topk_idx=topk,
                    num_experts=16, alignment=16, sr_seed=1234, sr_counter_base=0)


def config5(seed=0):
    """Grouped dSwiGLU: 8 experts with counts [0,512,3000,64,8192,1,2048,1024] (expert-major rows),
    preact [T, 2*2048] ~ N(0,1), dy [T, 2048] ~ N(0, 1e-2^2)."""
    counts = np.array([0, 512, 3000, 64, 8192, 1, 2048, 1024], dtype=np.int32)
    t = int(counts.sum())
    r = _streams(seed, 2)
    pre = r[0].standard_normal((t, 4096), dtype=np.float32)
    dy = r[1].standard_normal((t, 2048), dtype=np.float32) * np.float32(1e-2)
    return Workload("dswiglu-fc1grad-14841x2x2048-e8", preact_bits=to_bf16_bits(pre),
                    dy_bits=to_bf16_bits(dy), counts=counts, num_experts=8, alignment=16)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def small_dispatch(seed, tokens, hidden, num_experts, top_k, alignment=16, scale=1.0,
                   unused_frac=0.0, empty=()):
    """A small random dispatch case for parity sweeps (ragged shapes, -1 slots, empty experts)."""
    r = _streams(seed, 4)
    x = r[0].standard_normal((tokens, hidden)) * scale
    mag = 10.0 ** r[1].uniform(-1.0, 1.0, size=(tokens, 1))
    x = x * mag
    experts = [e for e in range(num_experts) if e not in set(empty)]
    if top_k > len(experts):
        raise ValueError("top_k larger than the non-empty expert count")
    logits = r[2].standard_normal((tokens, len(experts)))
    topk = np.array(experts, dtype=np.int32)[np.argsort(-logits, axis=1, kind="stable")[:, :top_k]]
    if unused_frac > 0:
        topk = np.where(r[3].random(topk.shape) < unused_frac, -1, topk).astype(np.int32)
    return Workload(f"small-{tokens}x{hidden}-e{num_experts}-k{top_k}", x_bits=to_bf16_bits(x),
                    topk_idx=topk.astype(np.int32), num_experts=num_experts, alignment=alignment)


def small_dswiglu(seed, counts, ffn, dy_scales=None):
    """A small grouped dSwiGLU case; dy_scales (one per expert) rescale each expert's dy rows."""
    counts = np.asarray(counts, dtype=np.int32)
    t = int(counts.sum())
    r = _streams(seed, 2)
    pre = r[0].standard_normal((t, 2 * ffn))
    dy = r[1].standard_normal((t, ffn)) * 1e-2
    if dy_scales is not None:
        dy = dy * np.repeat(np.asarray(dy_scales, dtype=np.float64), counts)[:, None]
    return Workload(f"small-dswiglu-{t}x{ffn}", preact_bits=to_bf16_bits(pre), dy_bits=to_bf16_bits(dy),
                    counts=counts, num_experts=len(counts))
