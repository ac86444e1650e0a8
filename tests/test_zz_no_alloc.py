"""moe_wna16_forward_noalloc: the layer without a caller workspace, on the
library's per-GPU scratch array, called through the C ABI.

Two calls in a row per case, the second with a smaller batch on the same
scratch.  Each output is compared with moe_wna16_forward's on the same inputs
(whose FP32 sum run_layer checks against the oracle within the tolerance, and
whose BF16 output is the rounding of that sum) and with the oracle directly:
  - top-1 routing: one contribution per output element, so no atomic order
    enters and the two entry points must agree bit for bit;
  - top-k > 1: the FP32 atomics add a token's k contributions in either order,
    so the two roundings may differ by one BF16 unit in the last place; the
    no-alloc output must lie within the tolerance plus half a BF16 unit of the
    oracle (the rounding of a sum that meets the tolerance).
"""
import math

import numpy as np
import pytest
import torch

import weight_only_bit_moe_amd as M
from oracle import oracle as O
from tests import _gpu as G
from weight_only_bit_moe_amd.inputs import CONFIGS, LayerSpec, make_config, make_layer, shard_spec

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="noalloc", T=8, H=256, I=128, E=8, topk=2, bits13=4, group13=128, bits2=4,
                group2=128, scale_lo=0.005, scale_hi=0.02)
    base.update(kw)
    return LayerSpec(**base)


def first_tokens(L, T):
    """The same layer with only its first T tokens (weights shared)."""
    import dataclasses
    return dataclasses.replace(L, spec=L.spec.replace(T=T), x=L.x[:T].copy(),
                               topk_ids=L.topk_ids[:T].copy(), topk_w=L.topk_w[:T].copy())


def noalloc(L, d, dev):
    sp = L.spec
    out = torch.full((sp.T, sp.H), 7.0, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = M.moe_wna16_forward_noalloc(
        d["x"].data_ptr(), d["topk_ids"].data_ptr(), d["topk_w"].data_ptr(), d["w13"].data_ptr(),
        d["s13"].data_ptr(), d["w2"].data_ptr(), d["s2"].data_ptr(), sp.T, sp.H, sp.I, sp.E,
        sp.topk, (sp.bits13, sp.group13), (sp.bits2, sp.group2), sp.alpha, sp.beta, sp.clamp,
        out.data_ptr(), stream)
    assert st == 0, M.moe_wna16_status_string(st)
    torch.cuda.synchronize(dev)
    return out


def bf16_ulp(v):
    """One BF16 unit in the last place at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_pair(L, dev):
    sp = L.spec
    d = G.to_device(L, dev)
    y_n = G.to_f64(noalloc(L, d, dev))
    y_f, f32 = G.run_layer(L, dev, d)
    ref = O.forward_layer(L)
    G.assert_parity(f32, ref, f"{sp.name} forward")
    y_f = G.to_f64(y_f)
    if sp.topk == 1:
        assert np.array_equal(y_n, y_f), "top-1: no-alloc output differs from forward's"
    else:
        diff = np.abs(y_n - y_f)
        assert np.all(diff <= bf16_ulp(np.maximum(np.abs(y_n), np.abs(y_f)))), \
            "no-alloc and forward outputs differ by more than one BF16 unit"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = G.REL * rms + G.ABS + 0.5 * bf16_ulp(y_n)
    assert np.all(np.abs(y_n - ref) <= bound), f"{sp.name}: no-alloc output outside the bound"


CASES = {
    # the decode workload at full size (the whole layer in one launch), then 2 tokens
    "decode_w2g128_full": (lambda: make_config(2), 2),
    # one GPU's share under tensor parallelism 4 (I = 512): the single launch
    # with gate/up items split over K slices and their partial-sum buffer
    "decode_tp4_share": (lambda: make_layer(shard_spec(2, "tp4"), 2), 2),
    # top-1: bit-exact against forward; decode-shaped, separate launches
    "decode_top1": (lambda: make_layer(spec(T=12, H=512, I=256, E=16, topk=1, bits13=2,
                                            bits2=2), seed=5), 5),
    # prefill-shaped plan (64-row tiles, XCD split) that fits the scratch
    "prefill_small": (lambda: make_layer(spec(T=96, H=256, I=256, E=4, topk=2, group13=64,
                                              bits2=2, group2=64, routing="zipf",
                                              alpha=1.702, beta=1.0, clamp=7.0), seed=6), 40),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_matches_forward_two_calls(name):
    dev = G.device()
    make, t_small = CASES[name]
    L = make()
    print(f"noalloc case {name}: T={L.spec.T} then {t_small}", flush=True)
    check_pair(L, dev)
    check_pair(first_tokens(L, t_small), dev)


def test_noalloc_rejects_calls_beyond_the_scratch():
    """The 2048-token prefill workload needs far more than 32 MiB: ESCRATCH,
    before any launch (the output keeps its contents)."""
    dev = G.device()
    sp = CONFIGS[4]
    x = torch.zeros((sp.T, sp.H), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((sp.T, sp.topk), dtype=torch.int32, device=dev)
    w = torch.zeros((sp.T, sp.topk), dtype=torch.float32, device=dev)
    codes = torch.zeros(16, dtype=torch.int32, device=dev)
    scales = torch.zeros(16, dtype=torch.float16, device=dev)
    out = torch.full((sp.T, sp.H), 3.0, dtype=torch.bfloat16, device=dev)
    st = M.moe_wna16_forward_noalloc(
        x.data_ptr(), ids.data_ptr(), w.data_ptr(), codes.data_ptr(), scales.data_ptr(),
        codes.data_ptr(), scales.data_ptr(), sp.T, sp.H, sp.I, sp.E, sp.topk, (2, 128), (2, 128),
        1.0, 0.0, math.inf, out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize(dev)
    assert st == -7   # ESCRATCH
    assert bool((out == 3.0).all())
