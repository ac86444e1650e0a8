"""Seeded synthetic inputs for the routed WNA16 MoE layer.

This module only draws inputs.  It holds none of the layer's arithmetic: no
unpacking, no dequantization, no activation, no routing sums.  Both the CPU
oracle (through the tests) and the HIP library consume exactly the arrays built
here, so the two sides see identical bytes.

Workloads follow the pages' formats: symmetric 2-bit / 4-bit signed codes packed
into 32-bit words with one FP16 scale per K group (model card
"hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What changed"), fused gate/up (w13)
and down (w2) projections with their own bit width and group size (PR "Incubate
DeepSeek V4 WNA16 runtime on SM86", "What this branch adds" items 2 and 9, and
"Validation completed"), BF16 activations and top-k indexed routing (same PR,
item 3).

Codes are drawn as uniform random 32-bit words.  Every code field of a word is
then uniform over the full b-bit range, which is exactly the code
distribution the workloads ask for ([-2, 1] for 2-bit, [-8, 7] for 4-bit), and
it is so under any sign encoding of the field.

Draw order for one layer (fixed, so a seed names the bytes):
  1. routing ids   2. routing weights   3. x   4. outlier channels
  5. w13 words     6. w13 scales        7. w2 words   8. w2 scales
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Layer",
    "LayerSpec",
    "CONFIGS",
    "make_layer",
    "make_batch",
    "make_config",
    "SHARDS",
    "shard_spec",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "QuantSpec",
    "QUANT_WORKLOAD",
    "make_dense_weights",
    "make_dense_weights_device",
    "make_importance",
]


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape, format and distribution recipe of one synthetic layer."""

    name: str
    T: int
    H: int
    I: int
    E: int
    topk: int
    bits13: int
    group13: int
    bits2: int
    group2: int
    routing: str = "uniform"          # "uniform" | "zipf"
    zipf_s: float = 1.1
    scale_lo: float = 0.01
    scale_hi: float = 0.05
    scale_dist: str = "uniform"       # "uniform" | "loguniform"
    x_sigma: float = 1.0
    outlier_frac: float = 0.0         # fraction of hidden channels scaled up
    outlier_mult: float = 10.0
    alpha: float = 1.0
    beta: float = 0.0
    clamp: float = math.inf
    # experts the routing draws from (0: E).  With more than E, the layer is
    # one GPU's share of an expert-parallel layer: it holds experts [0, E)
    # and receives the tokens' global top-k ids, the others belonging to
    # other GPUs.
    routing_experts: int = 0

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class Layer:
    """Host arrays of one layer, in the boundary's layouts.

    x           uint16 [T, H]            bf16 bit patterns, row-major
    topk_ids    int32  [T, k]
    topk_w      float32[T, k]
    w13         uint32 [E, 2I, H*b13/32] rows 0..I-1 gate (w1), I..2I-1 up (w3)
    s13         float16[E, 2I, H/g13]
    w2          uint32 [E, H, I*b2/32]
    s2          float16[E, H, I/g2]
    """

    spec: LayerSpec
    x: np.ndarray
    topk_ids: np.ndarray
    topk_w: np.ndarray
    w13: np.ndarray
    s13: np.ndarray
    w2: np.ndarray
    s2: np.ndarray
    outlier_channels: np.ndarray

    @property
    def T(self):
        return self.spec.T

    @property
    def H(self):
        return self.spec.H

    @property
    def I(self):
        return self.spec.I

    @property
    def E(self):
        return self.spec.E

    @property
    def topk(self):
        return self.spec.topk


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns.  Inputs are finite by construction here.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _routing_ids(rng: np.random.Generator, spec: LayerSpec) -> np.ndarray:
    T, k = spec.T, spec.topk
    E = spec.routing_experts or spec.E
    if k > E:
        raise ValueError("distinct top-k routing needs topk <= E")
    if spec.routing == "uniform":
        # first k entries of an independent uniform permutation of the experts
        perms = rng.permuted(np.tile(np.arange(E, dtype=np.int64), (max(T, 1), 1)), axis=1)[:T]
        return perms[:, :k].astype(np.int32)
    if spec.routing == "zipf":
        # expert of popularity rank r (1-based) has probability proportional to
        # r**-s; ranks are assigned through a seeded permutation of the experts.
        perm = rng.permutation(E)
        logp = np.empty(E, dtype=np.float64)
        logp[perm] = -spec.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        # k distinct draws without replacement: Gumbel top-k on log p
        keys = logp[None, :] + rng.gumbel(size=(T, E))
        order = np.argsort(-keys, axis=1, kind="stable")
        return order[:, :k].astype(np.int32)
    raise ValueError(f"unknown routing {spec.routing!r}")


def _scales(rng: np.random.Generator, spec: LayerSpec, shape) -> np.ndarray:
    if spec.scale_dist == "uniform":
        s = rng.uniform(spec.scale_lo, spec.scale_hi, size=shape)
    elif spec.scale_dist == "loguniform":
        s = np.exp(rng.uniform(math.log(spec.scale_lo), math.log(spec.scale_hi), size=shape))
    else:
        raise ValueError(spec.scale_dist)
    return s.astype(np.float16)  # float64 -> float16, round to nearest even


def _draw_batch(rng: np.random.Generator, spec: LayerSpec, outlier_channels=None):
    """Draws 1-4 of the fixed order: routing ids, routing weights, x, outliers."""
    T, H, k = spec.T, spec.H, spec.topk
    ids = _routing_ids(rng, spec) if T > 0 else np.zeros((0, k), np.int32)
    logits = rng.standard_normal((T, k))
    if T > 0:
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    else:
        w = logits.astype(np.float32)
    xf = (rng.standard_normal((T, H)) * spec.x_sigma).astype(np.float32)
    n_out = int(round(spec.outlier_frac * H))
    if n_out > 0:
        drawn = np.sort(rng.choice(H, size=n_out, replace=False))
        out_ch = drawn if outlier_channels is None else np.asarray(outlier_channels)
        xf[:, out_ch] *= np.float32(spec.outlier_mult)
    else:
        out_ch = np.zeros(0, np.int64)
    return ids, w, f32_to_bf16_bits(xf), out_ch.astype(np.int64)


def make_batch(spec: LayerSpec, seed: int, outlier_channels=None):
    """A fresh batch (topk_ids, topk_w, x) of the workload's distributions for an
    existing layer; pass the layer's outlier channels to keep them fixed."""
    ids, w, x, _ = _draw_batch(np.random.default_rng(seed), spec, outlier_channels)
    return ids, w, x


def make_layer(spec: LayerSpec, seed: int, topk_ids: Optional[np.ndarray] = None) -> Layer:
    """Draw one layer.  `topk_ids`, when given, replaces the routing draw
    (the routing-id draws are still made so the other arrays keep their bytes)."""
    T, H, I, E, k = spec.T, spec.H, spec.I, spec.E, spec.topk
    rng = np.random.default_rng(seed)
    ids, w, x, out_ch = _draw_batch(rng, spec)
    if topk_ids is not None:
        ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(T, k)
    w13 = rng.integers(0, 2**32, size=(E, 2 * I, H * spec.bits13 // 32), dtype=np.uint32)
    s13 = _scales(rng, spec, (E, 2 * I, H // spec.group13))
    w2 = rng.integers(0, 2**32, size=(E, H, I * spec.bits2 // 32), dtype=np.uint32)
    s2 = _scales(rng, spec, (E, H, I // spec.group2))
    return Layer(spec, x, ids, w, w13, s13, w2, s2, out_ch)


_BIG = dict(H=4096, I=2048, E=256)

#: The five named workloads.  Values follow the configuration list this project
#: measures on; where a workload leaves a distribution unstated it reuses the
#: closest stated one (prefill-chunk codes and scales as in the decode W2 layer).
CONFIGS = {
    1: LayerSpec("tiny-w4g128-T8", T=8, H=256, I=128, E=8, topk=2, bits13=4, group13=128,
                 bits2=4, group2=128, routing="uniform", scale_lo=0.005, scale_hi=0.02),
    2: LayerSpec("decode-w2g128-T4", T=4, **_BIG, topk=6, bits13=2, group13=128, bits2=2,
                 group2=128, routing="uniform", scale_lo=0.01, scale_hi=0.05),
    3: LayerSpec("batched-decode-w4g128-T64", T=64, **_BIG, topk=6, bits13=4, group13=128,
                 bits2=4, group2=128, routing="uniform", scale_lo=0.002, scale_hi=0.01),
    4: LayerSpec("prefill-w2g128-T2048-zipf", T=2048, **_BIG, topk=6, bits13=2, group13=128,
                 bits2=2, group2=128, routing="zipf", scale_lo=0.01, scale_hi=0.05,
                 alpha=1.702, beta=1.0, clamp=7.0),
    5: LayerSpec("prefill-w4g128-w2g64-T8192-zipf", T=8192, **_BIG, topk=8, bits13=4,
                 group13=128, bits2=2, group2=64, routing="zipf", scale_lo=1e-3, scale_hi=5e-2,
                 scale_dist="loguniform", x_sigma=2.0, outlier_frac=0.01, alpha=1.702,
                 beta=1.0, clamp=7.0),
}


#: One GPU's share of the decode and prefill-chunk workloads when the layer is
#: sharded: expert parallelism over 8 GPUs (32 local experts, the routing over
#: all 256) and tensor parallelism over 4 (intermediate 512 of 2048 per GPU:
#: its slice of every expert's gate, up and down rows).
SHARDS = {
    "ep8": dict(E=32, routing_experts=256),
    "tp4": dict(I=512),
}


def shard_spec(idx: int, shard: str) -> LayerSpec:
    sp = CONFIGS[idx]
    return sp.replace(name=f"{sp.name}-{shard}", **SHARDS[shard])


def make_config(idx: int, seed: Optional[int] = None) -> Layer:
    """Layer of named workload `idx` (1..5); the seed defaults to `idx`."""
    return make_layer(CONFIGS[idx], idx if seed is None else seed)


# ---- dense weights for the quantizer -----------------------------------------
#
# The quantizer's inputs (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16",
# "How it was created": routed-expert matrices and an activation importance
# vector per input channel).  The real matrices and importance data are not
# available, so:
#   weights    Student-t with 4 degrees of freedom times `w_std`, rounded to
#              BF16 (heavy tails give groups with a few large weights, the case
#              a scale search exists for).  t4 = z / sqrt(chi2_4 / 4) with
#              chi2_4 = -2 ln(U1 U2).
#   importance lognormal exp(sigma * z) per input channel, and a fraction
#              `outlier_frac` of channels multiplied by outlier_mult^2 (the mean
#              squared activation of a channel that runs outlier_mult times
#              hotter).

@dataclasses.dataclass(frozen=True)
class QuantSpec:
    """One quantizer workload: `matrices` of [rows, K] each."""

    name: str
    rows: int
    K: int
    bits: int
    group: int
    ncand: int
    matrices: int = 1
    w_std: float = 0.02
    imp_sigma: float = 1.0
    outlier_frac: float = 0.01
    outlier_mult: float = 10.0


#: All routed experts of one layer in the 2-bit, group-128 format: the fused
#: gate/up matrices of 256 experts as one [256 * 4096, 4096] operand and the
#: down matrices as one [256 * 4096, 2048] operand, with a 16-point scale search.
QUANT_WORKLOAD = (
    QuantSpec("quantize-w13-E256-w2g128-C16", rows=256 * 4096, K=4096, bits=2, group=128,
              ncand=16),
    QuantSpec("quantize-w2-E256-w2g128-C16", rows=256 * 4096, K=2048, bits=2, group=128,
              ncand=16),
)


def make_dense_weights(rows: int, K: int, seed: int, w_std: float = 0.02) -> np.ndarray:
    """Host draw: BF16 bit patterns [rows, K] of w_std * t4."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, K))
    u = rng.random((2, rows, K))
    t = z / np.sqrt(-0.5 * np.log(u[0] * u[1] + 1e-300))
    return f32_to_bf16_bits((t * w_std).astype(np.float32))


def make_dense_weights_device(rows: int, K: int, seed: int, device, w_std: float = 0.02,
                              chunk_rows: int = 1 << 15):
    """Device draw of the same distribution (torch's generator, so other bytes
    than the host draw): a BF16 tensor [rows, K] on `device`, made in chunks."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((rows, K), dtype=torch.bfloat16, device=device)
    for r0 in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r0)
        z = torch.randn((n, K), generator=g, device=device)
        u = torch.rand((2, n, K), generator=g, device=device)
        t = z / torch.sqrt(-0.5 * torch.log(u[0] * u[1] + 1e-30))
        out[r0:r0 + n] = (t * w_std).to(torch.bfloat16)
    return out


def make_importance(K: int, seed: int, sigma: float = 1.0, outlier_frac: float = 0.01,
                    outlier_mult: float = 10.0) -> np.ndarray:
    """Importance per input channel, float32 [K], all > 0."""
    rng = np.random.default_rng(seed)
    imp = np.exp(sigma * rng.standard_normal(K))
    n_out = int(round(outlier_frac * K))
    if n_out:
        imp[rng.choice(K, size=n_out, replace=False)] *= outlier_mult ** 2
    return imp.astype(np.float32)
