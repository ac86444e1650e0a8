"""Pins of the oracle's routed layer.

out[t] = sum_j w[t][j] * W2_e * SwiGLU(W13_e x_t), e = ids[t][j]: fused gate/up
(w13) and down (w2) projections with their own WNA16 schemas over BF16
indexed-MoE activations (PR "Incubate DeepSeek V4 WNA16 runtime on SM86",
"What this branch adds" items 2, 3 and 9; model card
"hampsonw/DeepSeek-V4-Flash-0731-WNA16", "What changed").

Pinned against: a dense brute force written separately (every expert for every
token, weight 0 where not routed), closed forms, and invariants of the
definition (token permutation, expert renaming, linearity in the routing
weights).
"""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests import _brute as B
from weight_only_bit_moe_amd.inputs import LayerSpec, make_layer

INF = float("inf")


def tiny(**kw):
    base = dict(name="t", T=6, H=256, I=128, E=8, topk=2, bits13=4, group13=128, bits2=4,
                group2=128, scale_lo=0.005, scale_hi=0.02)
    base.update(kw)
    return LayerSpec(**base)


def rel_err(a, b):
    scale = max(np.sqrt(np.mean(b ** 2)), 1e-300)
    return np.max(np.abs(a - b)) / scale


CASES = [
    dict(),
    dict(bits13=2, bits2=2, group13=64, group2=64, scale_lo=0.01, scale_hi=0.05),
    dict(bits13=4, group13=32, bits2=2, group2=128, alpha=1.702, beta=1.0, clamp=7.0),
    dict(bits13=2, group13=128, bits2=4, group2=32, alpha=1.702, beta=1.0, clamp=0.05),
    dict(E=1, topk=1),
    dict(E=5, topk=5, T=3, H=128, I=256),
    dict(routing="zipf", T=9, topk=3, x_sigma=2.0, outlier_frac=0.05, scale_dist="loguniform",
         scale_lo=1e-3, scale_hi=5e-2, clamp=7.0, alpha=1.702, beta=1.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_dense_brute_force(case):
    L = make_layer(tiny(**CASES[case]), seed=100 + case)
    got = O.forward_layer(L)
    ref = B.dense_forward(L)
    assert got.shape == ref.shape
    assert rel_err(got, ref) < 1e-12


def test_single_expert_dense_glu_mlp():
    """E = 1, k = 1, w = 1 is a dense GLU MLP: W2 act(W13 x) by numpy matmul."""
    sp = tiny(E=1, topk=1, alpha=1.702, beta=1.0, clamp=7.0, scale_lo=0.02, scale_hi=0.05)
    L = make_layer(sp, seed=5)
    L.topk_w[:] = 1.0
    W13 = B.dequant(L.w13[0], L.s13[0], sp.H, sp.bits13, sp.group13)
    W2 = B.dequant(L.w2[0], L.s2[0], sp.I, sp.bits2, sp.group2)
    x = B.bf16_to_f64(L.x)
    h = x @ W13.T
    act = B.swiglu(h[:, :sp.I], h[:, sp.I:], sp.alpha, sp.beta, sp.clamp)
    ref = act @ W2.T
    assert rel_err(O.forward_layer(L), ref) < 1e-12


def _const_layer(H, I, q13_word, q2_word, scale, ids, w, alpha=1.0, beta=0.0, clamp=INF):
    """Layer whose every code and scale is constant per expert: closed form."""
    E = len(q13_word)
    T, k = ids.shape
    sp = LayerSpec("closed", T=T, H=H, I=I, E=E, topk=k, bits13=4, group13=H, bits2=4,
                   group2=I, alpha=alpha, beta=beta, clamp=clamp)
    L = make_layer(sp, seed=0, topk_ids=ids)
    L.topk_w[:] = np.asarray(w, np.float32)
    L.x[:] = 0x3F80                                    # bf16 1.0 everywhere
    for e in range(E):
        L.w13[e][:] = q13_word[e]
        L.w2[e][:] = q2_word[e]
    L.s13[:] = np.float16(scale)
    L.s2[:] = np.float16(scale)
    return L


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_closed_form_two_experts():
    """H = I = 8, x = 1, scale 1/2.  Expert 0 has every code +1 (field 9),
    expert 1 every code -1 (field 7).  Gate = up = +-4 after w13, so
    act0 = 4 sig(4) 4 = 16 sig(4), act1 = (-4) sig(-4) (-4) = 16 sig(-4); w2 sums
    8 entries of +-1/2: y0 = 64 sig(4), y1 = -64 sig(-4).  With weights
    (1/4, 3/4): out = 16 sig(4) - 48 sig(-4) in every channel."""
    ids = np.array([[0, 1]], np.int32)
    L = _const_layer(8, 8, [0x99999999, 0x77777777], [0x99999999, 0x77777777], 0.5, ids,
                     [[0.25, 0.75]])
    out = O.forward_layer(L)
    expect = 16 * sig(4) - 48 * sig(-4)
    assert np.allclose(out, expect, rtol=1e-14, atol=0)


def test_closed_form_clamp_alpha_beta():
    """Same expert 0 with alpha = 1.702, beta = 1, clamp 3: gate and up (= 4)
    both clamp to 3, act = 3 sig(1.702*3) (3 + 1); y = 8 * act / 2."""
    ids = np.array([[0]], np.int32)
    L = _const_layer(8, 8, [0x99999999], [0x99999999], 0.5, ids, [[1.0]], alpha=1.702,
                     beta=1.0, clamp=3.0)
    out = O.forward_layer(L)
    act = 3 * sig(1.702 * 3) * 4
    assert np.allclose(out, 4 * act, rtol=1e-14, atol=0)


def test_token_permutation_permutes_output():
    L = make_layer(tiny(T=7), seed=21)
    base = O.forward_layer(L)
    perm = np.random.default_rng(1).permutation(7)
    L.x, L.topk_ids, L.topk_w = L.x[perm].copy(), L.topk_ids[perm].copy(), L.topk_w[perm].copy()
    assert np.array_equal(O.forward_layer(L), base[perm])


def test_expert_renaming_is_invisible():
    L = make_layer(tiny(T=5, E=6, topk=3), seed=22)
    base = O.forward_layer(L)
    pi = np.random.default_rng(2).permutation(6)          # new name of expert e is pi[e]
    inv = np.argsort(pi)
    L.topk_ids = pi[L.topk_ids].astype(np.int32)
    L.w13, L.s13, L.w2, L.s2 = L.w13[inv].copy(), L.s13[inv].copy(), L.w2[inv].copy(), L.s2[inv].copy()
    assert np.array_equal(O.forward_layer(L), base)


def test_linear_in_routing_weights():
    L = make_layer(tiny(T=4, topk=3), seed=23)
    base = O.forward_layer(L)
    L.topk_w = (L.topk_w * 2).astype(np.float32)
    assert np.array_equal(O.forward_layer(L), 2 * base)
    # one slot at a time sums to the whole (up to rounding order)
    parts = []
    w = L.topk_w.copy()
    for j in range(3):
        L.topk_w = np.zeros_like(w)
        L.topk_w[:, j] = w[:, j]
        parts.append(O.forward_layer(L))
    assert rel_err(sum(parts), 2 * base) < 1e-13


def test_zero_weight_and_out_of_range_ids_contribute_nothing():
    L = make_layer(tiny(T=4, topk=3), seed=24)
    L.topk_w[:, 2] = 0.0
    a = O.forward_layer(L)
    L.topk_ids[:, 2] = -1
    b = O.forward_layer(L)
    L.topk_ids[:, 2] = L.E + 3
    c = O.forward_layer(L)
    assert np.array_equal(a, b) and np.array_equal(b, c)


def test_duplicate_ids_sum():
    L = make_layer(tiny(T=3, topk=2), seed=25)
    L.topk_ids[:, 1] = L.topk_ids[:, 0]
    a = O.forward_layer(L)
    L2 = make_layer(tiny(T=3, topk=2), seed=25)
    L2.topk_ids[:, 1] = -1
    L2.topk_ids[:, 0] = L.topk_ids[:, 0]
    L2.topk_w[:, 0] = L.topk_w[:, 0] + L.topk_w[:, 1]
    assert rel_err(a, O.forward_layer(L2)) < 1e-6   # float32 sum of the two weights


def test_token_subset_rows_match_full_layer():
    L = make_layer(tiny(T=6), seed=26)
    full = O.forward_layer(L)
    sub = O.forward_layer(L, tokens=[4, 0, 4])
    assert np.array_equal(sub, full[[4, 0, 4]])


def test_empty_batch():
    L = make_layer(tiny(T=0), seed=27)
    assert O.forward_layer(L).shape == (0, 256)
