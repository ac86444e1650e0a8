"""GPU parity on seeded random layer shapes (tests/_random_shapes.py).

Each case draws the token count, hidden and intermediate sizes (multiples of
128), the expert count and top-k, the bit width and group size of each
projection, the routing (uniform or Zipf) and the activation parameters from
its own seed; the plan then picks the decode-shaped, single-launch or
prefill-shaped path by itself.  Every case is compared with the oracle on all
of its tokens (the tolerance, the BF16 rounding, the fused-wait status and
the layer's own sort are checked as in the fixed cases), sizes being capped
so that the oracle finishes in about a second.  Prefill-shaped plans also
check the XCD split they ran against the host model, and decode-shaped ones
run a second time on prepared codes.
"""
import pytest

import weight_only_bit_moe_amd as M
from oracle import oracle as O
from tests import _gpu as G
from tests._random_shapes import LARGE_SEEDS, SEEDS, random_large_spec, random_spec
from weight_only_bit_moe_amd.inputs import make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return G.device()


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_matches_oracle(dev, seed):
    sp = random_spec(seed)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    print(f"{sp.name}: T={sp.T} H={sp.H} I={sp.I} E={sp.E} k={sp.topk} "
          f"w13=W{sp.bits13}g{sp.group13} w2=W{sp.bits2}g{sp.group2} {sp.routing} "
          f"plan={plan}", flush=True)
    L = make_layer(sp, seed=seed)
    ref = O.forward_layer(L)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    _, got = G.run_layer(L, dev, workspace=ws)
    G.assert_parity(got, ref, sp.name)
    if plan["w13_variant"] == 1:
        G.assert_xcd_split(L, ws)
    if plan["w13_variant"] == 2 and plan["w2_variant"] == 2:
        _, got_p = G.run_layer(L, dev, prepared=True)
        G.assert_parity(got_p, ref, sp.name + " prepared")


@pytest.mark.parametrize("seed", LARGE_SEEDS)
def test_random_large_shape_sampled_tokens(dev, seed):
    """Realistic sizes (hidden up to 4096, intermediate up to 2048, up to
    4095 tokens), checked on 12 tokens the oracle computes one by one: the
    tiles on both sides of the XCD range boundaries, the first and last
    tile, the least-used experts' tokens."""
    sp = random_large_spec(seed)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    print(f"{sp.name}: T={sp.T} H={sp.H} I={sp.I} E={sp.E} k={sp.topk} "
          f"w13=W{sp.bits13}g{sp.group13} w2=W{sp.bits2}g{sp.group2} {sp.routing} "
          f"plan={plan}", flush=True)
    L = make_layer(sp, seed=seed)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    _, got = G.run_layer(L, dev, workspace=ws)
    rows = G.sampled_tokens(L, ws, n=12)
    G.assert_parity(got[rows], O.forward_layer(L, tokens=rows), sp.name)
    if plan["w13_variant"] == 1:
        G.assert_xcd_split(L, ws)
