"""Seeded random layer shapes for the random-shape parity tests."""
import math

import numpy as np

from weight_only_bit_moe_amd.inputs import LayerSpec

#: multiply-adds the oracle may spend on one case (about a second)
MAX_MACS = 3e8
SEEDS = range(96)


def random_spec(seed: int) -> LayerSpec:
    """Seeds cycle through three draws: a prefill-sized batch (9-399 tokens),
    a decode-sized one (1-8 tokens) with any formats, and a decode-sized one
    (1-16 tokens, at least 16 experts) with one format on both projections,
    a hidden size of 1024 or 2048 and an intermediate of 512 or 1024 (the
    shapes the shared and single decode launches take)."""
    rng = np.random.default_rng(1000 + seed)
    mode = seed % 3
    if mode == 2:   # whole rounds of the shared launch's prefetch depth
        H = int(rng.choice([1024, 2048]))
        I = int(rng.choice([512, 1024]))
    else:
        H = 128 * int(rng.integers(1, 9))
        I = 128 * int(rng.integers(1, 9))
    E = int(rng.choice([16, 33, 64, 256] if mode == 2 else [1, 2, 3, 4, 8, 16, 33, 64, 256]))
    topk = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(9, 400)) if mode == 0 else int(rng.integers(1, 17 if mode == 2 else 9))
    T = max(1, min(T, int(MAX_MACS / (3.0 * H * I * topk))))
    bits13, bits2 = (int(rng.choice([2, 4])) for _ in range(2))
    group13, group2 = (int(rng.choice([32, 64, 128])) for _ in range(2))
    if mode == 2:
        bits13, group13 = [(2, 64), (2, 128), (4, 32), (4, 64), (4, 128)][int(rng.integers(0, 5))]
        bits2, group2 = bits13, group13
    act = rng.random() < 0.5
    return LayerSpec(
        name=f"random{seed}", T=T, H=H, I=I, E=E, topk=topk, bits13=bits13, group13=group13,
        bits2=bits2, group2=group2, routing="zipf" if rng.random() < 0.5 else "uniform",
        scale_lo=0.005, scale_hi=0.03,
        alpha=1.702 if act else 1.0, beta=1.0 if act else 0.0,
        clamp=7.0 if act else math.inf)

#: seeds of the realistic-size draws (checked on sampled tokens)
LARGE_SEEDS = range(12)
#: weight elements of one layer (E x 3 x H x I) the draws stay under
MAX_WEIGHTS = 1.6e9


def random_large_spec(seed: int) -> LayerSpec:
    """A prefill-sized layer of realistic shape: hidden 1024-4096,
    intermediate 512-2048, 16-256 experts (fewer when the weights would pass
    MAX_WEIGHTS elements), top-1 to top-8, 256-4095 tokens, any formats."""
    rng = np.random.default_rng(5000 + seed)
    H = int(rng.choice([1024, 2048, 4096]))
    I = int(rng.choice([512, 1024, 2048]))
    E = int(rng.choice([16, 32, 64, 128, 256]))
    while E > 16 and E * 3.0 * H * I > MAX_WEIGHTS:
        E //= 2
    topk = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(256, 4096))
    bits13, bits2 = (int(rng.choice([2, 4])) for _ in range(2))
    group13, group2 = (int(rng.choice([32, 64, 128])) for _ in range(2))
    act = rng.random() < 0.5
    return LayerSpec(
        name=f"random_large{seed}", T=T, H=H, I=I, E=E, topk=topk, bits13=bits13,
        group13=group13, bits2=bits2, group2=group2,
        routing="zipf" if rng.random() < 0.5 else "uniform", scale_lo=0.002, scale_hi=0.02,
        alpha=1.702 if act else 1.0, beta=1.0 if act else 0.0,
        clamp=7.0 if act else math.inf)
