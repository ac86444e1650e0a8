"""GPU parity of the prepared code order: moe_wna16_prepare against the
oracle's statement of the layout (bit for bit), and the layer through
moe_wna16_forward_prepared against the oracle (the same bound as the layer's
other parity tests), at small sizes and on sampled tokens of the full
decode-shaped workloads."""
import numpy as np
import pytest
import torch

import weight_only_bit_moe_amd as M
from oracle import oracle as O
from tests import _gpu as G
from weight_only_bit_moe_amd import binding as Bd
from weight_only_bit_moe_amd.inputs import LayerSpec, make_batch, make_config, make_layer

pytestmark = pytest.mark.gpu

FORMATS = [(2, 32), (2, 64), (2, 128), (4, 32), (4, 64), (4, 128)]


@pytest.fixture(scope="module")
def dev():
    return G.device()


@pytest.mark.parametrize("bits,group", FORMATS)
def test_prepare_matches_oracle(dev, bits, group):
    """3 experts x 48 rows x 1024 columns: several blocks and units each."""
    rng = np.random.default_rng(bits * 1000 + group)
    E, rows, K = 3, 48, 1024
    w = rng.integers(0, 2 ** 32, size=(E, rows, K * bits // 32), dtype=np.uint32)
    got = M.prepare(torch.from_numpy(w.view(np.int32)).to(dev), bits, group)
    torch.cuda.synchronize(dev)
    ref = O.prepare(w, bits, group)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref)


@pytest.mark.parametrize("bits,group,E,rows,K", [(4, 128, 1, 16, 128), (2, 32, 1, 16, 256),
                                                 (2, 128, 2, 16, 256)])
def test_prepare_single_block(dev, bits, group, E, rows, K):
    """One block per expert (16 rows x one load unit)."""
    rng = np.random.default_rng(E * rows + K + bits)
    w = rng.integers(0, 2 ** 32, size=(E, rows, K * bits // 32), dtype=np.uint32)
    got = M.prepare(torch.from_numpy(w.view(np.int32)).to(dev), bits, group)
    torch.cuda.synchronize(dev)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), O.prepare(w, bits, group))


def spec(**kw):
    base = dict(name="case", T=8, H=256, I=256, E=8, topk=2, bits13=4, group13=128, bits2=4,
                group2=128, scale_lo=0.005, scale_hi=0.02)
    base.update(kw)
    return LayerSpec(**base)


ACT = dict(alpha=1.702, beta=1.0, clamp=7.0)
CASES = {
    # one shared launch (same format on both projections)
    "w2g128_one_launch": spec(T=4, H=1024, I=512, E=8, topk=3, bits13=2, bits2=2),
    "w4g64_one_launch": spec(T=6, H=512, I=1024, E=16, topk=2, group13=64, group2=64, **ACT),
    "w4g32_one_launch": spec(T=5, H=512, I=256, E=6, topk=2, group13=32, group2=32),
    "w2g64_one_launch": spec(T=3, H=1024, I=512, E=4, topk=2, bits13=2, bits2=2, group13=64,
                             group2=64),
    # 2-bit g128, K of 2048 on both projections (several pipeline rounds)
    "w2g128_k2048_one_launch": spec(T=4, H=2048, I=2048, E=8, topk=3, bits13=2, bits2=2),
    "w2g128_w4g128_down": spec(T=5, H=2048, I=1024, E=8, topk=2, bits13=2, bits2=4, **ACT),
    # separate launches (formats differ, or 2-bit group 32)
    "w4g128_w2g64": spec(T=8, H=512, I=512, E=16, topk=4, bits2=2, group2=64, **ACT),
    "w2g32_w4g32": spec(T=6, H=512, I=256, E=8, topk=2, bits13=2, group13=32, group2=32),
    "w2g32_both": spec(T=4, H=256, I=512, E=8, topk=2, bits13=2, group13=32, bits2=2,
                       group2=32),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_forward_prepared_matches_oracle(dev, name):
    sp = CASES[name]
    L = make_layer(sp, seed=sum(map(ord, name)))
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    assert plan["w13_variant"] == 2 and plan["w2_variant"] == 2
    _, got = G.run_layer(L, dev, prepared=True)
    ref = O.forward_layer(L)
    G.assert_parity(got, ref, name)
    # the same kernels on the checkpoint order agree within the same bound
    _, plain = G.run_layer(L, dev)
    G.assert_parity(plain, ref, name + " (packed)")


@pytest.mark.parametrize("cfg", [2, 3])
def test_forward_prepared_full_workload_sampled_tokens(dev, cfg):
    L = make_config(cfg)
    print(f"prepared config {cfg} {L.spec.name}", flush=True)
    _, y = G.run_layer(L, dev, prepared=True)
    assert np.all(np.isfinite(y))
    rows = [0, 1, L.spec.T - 1] if L.spec.T > 3 else list(range(L.spec.T))
    G.assert_parity(y[rows], O.forward_layer(L, tokens=rows), f"config {cfg} prepared")


def test_forward_prepared_new_batches_on_one_workspace(dev):
    """Codes prepared once, then calls with a new routing batch each on one
    workspace and one output buffer (the shared decode launch with the fused
    rounding): every call matches the oracle."""
    sp = spec(T=4, H=1024, I=1024, E=16, topk=4, bits13=2, bits2=2)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (2, 128), (2, 128))
    assert plan["gemms_one_launch"] == 1 and plan["convert_in_w2"] == 1
    L = make_layer(sp, seed=77)
    d = G.to_device(L, dev)
    w13 = M.prepare(d["w13"], sp.bits13, sp.group13)
    w2 = M.prepare(d["w2"], sp.bits2, sp.group2)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    out = torch.empty((sp.T, sp.H), dtype=torch.bfloat16, device=dev)
    for rep in range(5):
        ids, w, x = make_batch(sp, seed=500 + rep)
        y = M.forward(torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16),
                      torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev), w13, d["s13"],
                      w2, d["s2"], bits=(sp.bits13, sp.bits2), group=(sp.group13, sp.group2),
                      alpha=sp.alpha, beta=sp.beta, clamp=None, out=out, workspace=ws,
                      prepared=True)
        torch.cuda.synchronize(dev)
        Lr = make_layer(sp, seed=77, topk_ids=ids)
        Lr.topk_w, Lr.x = w, x
        G.assert_parity(G.to_f64(y), O.forward_layer(Lr), f"batch {rep}")


def test_forward_prepared_rejects_prefill_shapes(dev):
    """64-row tiles read the checkpoint order only: EUNSUPPORTED, nothing launched."""
    sp = spec(T=64, H=256, I=256, E=4, topk=2)
    L = make_layer(sp, seed=3)
    d = G.to_device(L, dev)
    out = torch.full((sp.T, sp.H), 7.0, dtype=torch.bfloat16, device=dev)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    st = M.moe_wna16_forward_prepared(
        d["x"].data_ptr(), d["topk_ids"].data_ptr(), d["topk_w"].data_ptr(), d["w13"].data_ptr(),
        d["s13"].data_ptr(), d["w2"].data_ptr(), d["s2"].data_ptr(), sp.T, sp.H, sp.I, sp.E,
        sp.topk, (4, 128), (4, 128), 1.0, 0.0, float("inf"), out.data_ptr(), ws.data_ptr(),
        ws.numel(), None)
    torch.cuda.synchronize(dev)
    assert st == Bd.EUNSUPPORTED
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("HI", [256, 1024])   # separate / shared decode launches
def test_forward_prepared_edge_ids(dev, HI):
    """Invalid, out-of-range and duplicate ids and an empty expert, on
    prepared codes."""
    sp = spec(T=10, H=HI, I=HI, topk=3, E=8)
    L = make_layer(sp, seed=177)
    ids = L.topk_ids.copy()
    ids[0, 1] = -1
    ids[1, 2] = 8
    ids[2, 0] = 1000
    ids[3, 1] = ids[3, 0]
    ids[ids == 5] = 6
    L.topk_ids = ids.astype(np.int32)
    _, got = G.run_layer(L, dev, prepared=True)
    G.assert_parity(got, O.forward_layer(L), "edge ids, prepared")


@pytest.mark.parametrize("HI", [256, 1024])
def test_forward_prepared_all_ids_invalid_writes_zeros(dev, HI):
    sp = spec(T=4, H=HI, I=HI, topk=2, E=8)
    L = make_layer(sp, seed=179)
    L.topk_ids[:, :] = -1
    out = torch.full((sp.T, sp.H), 3.0, dtype=torch.bfloat16, device=dev)
    y, got = G.run_layer(L, dev, out=out, prepared=True)
    assert not G.to_f64(y).any()
    G.assert_parity(got, O.forward_layer(L), "all ids invalid, prepared")


@pytest.mark.parametrize("T,E", [(4, 8), (40, 32)])
def test_forward_prepared_events_bracket_the_launches(dev, T, E):
    """With an event array the prepared entry records launch start/stop
    events in stream order: the whole layer as one launch (8 pairs), or the
    routing launch and one shared w13 + w2 launch (80 pairs)."""
    import ctypes

    from bench import Hip

    sp = spec(T=T, H=1024, I=1024, E=E, topk=2, bits13=2, bits2=2)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (2, 128), (2, 128))
    assert plan["gemms_one_launch"] == 1 and plan["convert_in_w2"] == 1
    assert plan["single_launch"] == (1 if T * 2 <= 64 else 0)
    L = make_layer(sp, seed=181)
    d = G.to_device(L, dev)
    w13 = M.prepare(d["w13"], 2, 128)
    w2 = M.prepare(d["w2"], 2, 128)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    out = torch.empty((sp.T, sp.H), dtype=torch.bfloat16, device=dev)
    hip = Hip()
    ev = (ctypes.c_void_p * 8)(*[hip.event() for _ in range(8)])
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = M.moe_wna16_forward_prepared(
        d["x"].data_ptr(), d["topk_ids"].data_ptr(), d["topk_w"].data_ptr(), w13.data_ptr(),
        d["s13"].data_ptr(), w2.data_ptr(), d["s2"].data_ptr(), sp.T, sp.H, sp.I, sp.E, sp.topk,
        (2, 128), (2, 128), 1.0, 0.0, float("inf"), out.data_ptr(), ws.data_ptr(), ws.numel(),
        stream, ev)
    assert st == Bd.OK
    torch.cuda.synchronize(dev)
    if plan["single_launch"]:
        assert hip.elapsed_ms(ev[0], ev[5]) >= 0.0  # the one launch
    else:
        assert hip.elapsed_ms(ev[0], ev[1]) >= 0.0  # route
        assert hip.elapsed_ms(ev[2], ev[5]) >= 0.0  # the shared w13 + w2 launch
        assert hip.elapsed_ms(ev[1], ev[2]) >= 0.0  # in stream order
    f32 = M.workspace_f32_sum(ws, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16),
                          G.f32_to_bf16_bits(f32))
    G.assert_parity(f32.astype(np.float64), O.forward_layer(L), "prepared, with events")
    for e in ev:
        hip.destroy(e)
