"""The layer captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: the
path records no memset nodes (the accumulator, counters and bias terms are
cleared by kernels), so every replay must match the oracle.  Each replay gets
fresh inputs copied into the captured buffers, and eager work and host
synchronisation run between replays."""
import math

import numpy as np
import pytest
import torch

import weight_only_bit_moe_amd as M
from oracle import oracle as O
from tests import _gpu as G
from weight_only_bit_moe_amd.inputs import LayerSpec, make_batch, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return G.device()


def spec(**kw):
    base = dict(name="graph", T=4, H=1024, I=512, E=16, topk=4, bits13=2, group13=128, bits2=2,
                group2=128, scale_lo=0.005, scale_hi=0.02)
    base.update(kw)
    return LayerSpec(**base)


CASES = {
    # 16 pairs: the whole layer as one launch
    "decode_shared_launch": (spec(), False),
    # the single launch with gate/up items split over 4 K slices
    "decode_single_split": (spec(H=4096, E=64, topk=6), False),
    # 80 pairs: the routing launch, then one shared w13 + w2 launch with the
    # BF16 rounding inside it
    "decode_shared_80_pairs": (spec(T=20, E=32), False),
    "decode_prepared": (spec(), True),
    # separate decode launches (different formats)
    "decode_two_formats": (spec(T=6, bits2=4, group2=64), False),
    # 64-row tiles and the convert kernel
    "prefill_tiles": (spec(T=96, E=4, topk=2, bits13=4, bits2=4), False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_oracle(dev, name):
    sp, prepared = CASES[name]
    L = make_layer(sp, seed=sum(map(ord, name)))
    d = G.to_device(L, dev)
    w13, w2 = d["w13"], d["w2"]
    if prepared:
        w13 = M.prepare(w13, sp.bits13, sp.group13)
        w2 = M.prepare(w2, sp.bits2, sp.group2)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    out = torch.empty((sp.T, sp.H), dtype=torch.bfloat16, device=dev)
    clamp = None if math.isinf(sp.clamp) else sp.clamp

    def layer():
        M.forward(d["x"], d["topk_ids"], d["topk_w"], w13, d["s13"], w2, d["s2"],
                  bits=(sp.bits13, sp.bits2), group=(sp.group13, sp.group2), alpha=sp.alpha,
                  beta=sp.beta, clamp=clamp, out=out, workspace=ws, prepared=prepared)

    # warm up on a side stream (first calls cache device properties), then capture
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize(dev)

    other_ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    for rep in range(4):
        ids, w, x = make_batch(sp, seed=1000 + rep)
        d["topk_ids"].copy_(torch.from_numpy(ids))
        d["topk_w"].copy_(torch.from_numpy(w))
        d["x"].copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize(dev)
        f32 = M.workspace_f32_sum(ws, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()
        bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(bits, G.f32_to_bf16_bits(f32)), f"replay {rep}: rounding"
        Lr = make_layer(sp, seed=sum(map(ord, name)), topk_ids=ids)
        Lr.topk_w, Lr.x = w, x
        G.assert_parity(f32.astype(np.float64), O.forward_layer(Lr), f"{name} replay {rep}")
        # eager work on another workspace between replays
        M.forward(d["x"], d["topk_ids"], d["topk_w"], w13, d["s13"], w2, d["s2"],
                  bits=(sp.bits13, sp.bits2), group=(sp.group13, sp.group2), alpha=sp.alpha,
                  beta=sp.beta, clamp=clamp, workspace=other_ws, prepared=prepared)
        torch.cuda.synchronize(dev)
    del graph
