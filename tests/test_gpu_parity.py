"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Alignment outputs must match bit for bit.  The layer's FP32 sum must satisfy
|gpu - oracle| <= 2e-2 * rms(oracle) + 1e-3 elementwise (rms over all compared
elements), and its BF16 output must be the RNE rounding of that sum.  Shapes straddle every tiling threshold: 16- and 64-row tiles,
experts with 15/16/17 and 64/65 rows, K chunks of 128/256/512, W2/W4 with
group 32/64/128 on each projection, empty experts, invalid and duplicate ids.
The four full-size workloads run in the same launch configuration as the
benchmark and are checked on tokens the oracle computes one by one.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import weight_only_bit_moe_amd as M
from oracle import oracle as O
from tests import _gpu as G
from weight_only_bit_moe_amd.inputs import (CONFIGS, LayerSpec, make_config, make_layer,
                                            shard_spec)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return G.device()


# --------------------------------------------------------------------------
# alignment: bit-exact
# --------------------------------------------------------------------------

def gpu_align(ids_np, E, bm, dev):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).to(dev)
    r = M.align(ids, E, bm)
    torch.cuda.synchronize(dev)
    n = int(r["num_tiles"][0])
    P = ids_np.size
    return dict(sorted_ids=r["sorted_ids"][: n * bm].cpu().numpy(),
                tile_expert=r["tile_expert"][:n].cpu().numpy(),
                expert_offsets=r["expert_offsets"].cpu().numpy(),
                inv_perm=r["inv_perm"][:P].cpu().numpy(), num_tiles=n,
                bad_ids=int(r["bad_ids"][0]))


assert_align_equal = G.assert_align_equal


def _align_cases():
    cases = []
    rng = np.random.default_rng(1234)
    for i in range(12):
        T = int(rng.integers(1, 3000))
        k = int(rng.integers(1, 9))
        E = int(rng.choice([1, 3, 8, 64, 256, 1000, 1024]))
        cases.append((f"fuzz{i}", rng.integers(0, E, size=(T, k)), E))
    ids = rng.integers(-3, 20, size=(300, 4))           # invalid ids mixed in
    cases.append(("bad_ids", ids, 16))
    cases.append(("one_hot_expert", np.full((1500, 2), 7), 256))
    cases.append(("max_experts", rng.integers(0, 1024, size=(4096, 8)), 1024))
    # several workgroups (4096 pairs each): invalid ids, exact and ragged chunk ends
    cases.append(("bad_ids_multi_block", rng.integers(-3, 20, size=(3000, 4)), 16))
    cases.append(("exact_two_chunks", rng.integers(0, 64, size=(1024, 8)), 64))
    cases.append(("chunk_plus_one", rng.integers(0, 8, size=(4097, 1)), 8))
    # up to 64 pairs: one wave sorts them (no workgroup barriers)
    for i, (T, k, E) in enumerate([(1, 1, 1), (4, 6, 256), (8, 8, 1024), (3, 7, 1000),
                                   (16, 4, 8), (64, 1, 3), (2, 5, 64)]):
        cases.append((f"wave_fuzz{i}", rng.integers(0, E, size=(T, k)), E))
    cases.append(("wave_bad_ids", rng.integers(-3, 20, size=(15, 4)), 16))
    cases.append(("wave_all_bad", np.full((4, 6), 300), 256))
    cases.append(("wave_one_expert_64", np.full((64, 1), 5), 8))
    cases.append(("wave_65_pairs", rng.integers(0, 4, size=(13, 5)), 4))   # block path
    return cases


@pytest.mark.parametrize("bm", [1, 4, 16, 64, 128])
@pytest.mark.parametrize("case", range(len(_align_cases())))
def test_align_bit_exact(dev, case, bm):
    name, ids, E = _align_cases()[case]
    assert_align_equal(gpu_align(ids, E, bm, dev), O.align(ids, E, bm))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_align_bit_exact_on_workload_routing(dev, cfg):
    sp = CONFIGS[cfg]
    ids = make_layer(sp.replace(H=128, I=128, E=sp.E), cfg).topk_ids   # same routing draw
    bm = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                          (sp.bits2, sp.group2))["block_m"]
    assert_align_equal(gpu_align(ids, sp.E, bm, dev), O.align(ids, sp.E, bm))


def test_align_empty_batch(dev):
    got = gpu_align(np.zeros((0, 4), np.int32), 8, 16, dev)
    assert got["num_tiles"] == 0 and not got["expert_offsets"].any()


def test_align_deterministic(dev):
    ids = np.random.default_rng(5).integers(0, 256, size=(2048, 6))
    first = gpu_align(ids, 256, 64, dev)
    for _ in range(20):
        assert_align_equal(gpu_align(ids, 256, 64, dev), first)


# --------------------------------------------------------------------------
# the layer at sizes the oracle computes in full
# --------------------------------------------------------------------------

def spec(**kw):
    base = dict(name="case", T=8, H=256, I=128, E=8, topk=2, bits13=4, group13=128, bits2=4,
                group2=128, scale_lo=0.005, scale_hi=0.02)
    base.update(kw)
    return LayerSpec(**base)


ACT = dict(alpha=1.702, beta=1.0, clamp=7.0)
DEC, PRE = 2, 1   # decode-shaped (4-row tiles) and prefill-shaped (64-row tiles) kernels
SMALL = {
    # decode-shaped: at most 4 rows per expert on average
    "dec_tiny_config": (CONFIGS[1], None, DEC),
    "dec_w2g128_w2g64_kc": (spec(T=8, H=512, I=256, E=16, topk=4, bits13=2, bits2=2, group2=64,
                                 scale_lo=0.01, scale_hi=0.05, **ACT), None, DEC),
    "dec_w4g32_w2g32_clamp_binds": (spec(T=8, H=384, I=512, E=12, topk=3, group13=32, bits2=2,
                                         group2=32, alpha=1.702, beta=1.0, clamp=0.5), None, DEC),
    "dec_w2g32_w4g64": (spec(T=6, H=256, I=256, E=5, topk=2, bits13=2, group13=32, bits2=4,
                             group2=64), None, DEC),
    "dec_w4g64_w4g32_k4096": (spec(T=3, H=4096, I=256, E=4, topk=2, group13=64, group2=32),
                              None, DEC),
    "dec_w2g128_long_k": (spec(T=4, H=2048, I=1024, E=8, topk=3, bits13=2, bits2=2,
                               scale_lo=0.01, scale_hi=0.05), None, DEC),
    # the route kernel sorts up to 64 pairs on one wave, more on a workgroup
    "dec_64_pairs_one_wave_sort": (spec(T=8, H=1024, I=1024, E=16, topk=8, bits13=2, bits2=2),
                                   None, DEC),
    "dec_65_pairs_workgroup_sort": (spec(T=13, H=256, I=256, E=20, topk=5, bits13=2, bits2=2),
                                    None, DEC),
    "dec_3_4_5_rows": (spec(T=12, H=256, I=128, E=8, topk=2), "345", DEC),
    # 2-bit codes with K an odd multiple of 128: the tile kernel takes these
    # small batches (the decode kernels need K in units of 256)
    "small_batch_w2_k384": (spec(T=4, H=384, I=640, E=8, topk=2, bits13=2, bits2=2), None, PRE),
    "dec_single_expert": (spec(T=4, E=1, topk=1), None, DEC),
    # prefill-shaped
    "pre_w2_g128_g64_kc512": (spec(T=16, H=512, I=256, topk=4, bits13=2, bits2=2, group2=64,
                                   scale_lo=0.01, scale_hi=0.05, **ACT), None, PRE),
    "pre_w4g32_w2g32_clamp_binds": (spec(T=24, H=384, I=512, E=6, topk=3, group13=32, bits2=2,
                                         group2=32, alpha=1.702, beta=1.0, clamp=0.5), None, PRE),
    "pre_w2g32_w4g64": (spec(T=12, H=256, I=256, E=5, topk=2, bits13=2, group13=32, bits2=4,
                             group2=64), None, PRE),
    "pre_zipf_multi_tile": (spec(T=256, H=256, I=256, E=8, topk=2, group13=64,
                                 routing="zipf", **ACT), None, PRE),
    "pre_65_rows_per_expert": (spec(T=130, H=384, I=128, E=4, topk=2), "65each", PRE),
    "pre_w2g64_outliers": (spec(T=200, H=512, I=256, E=8, topk=4, bits13=4, bits2=2,
                                group2=64, routing="zipf", scale_dist="loguniform",
                                scale_lo=1e-3, scale_hi=5e-2, x_sigma=2.0,
                                outlier_frac=0.01, **ACT), None, PRE),
    "pre_15_16_17_rows": (spec(T=40, H=256, I=128, E=8, topk=2), "151617", PRE),
    "pre_single_expert": (spec(T=5, E=1, topk=1), None, PRE),
    "pre_threshold_bm64_exact": (spec(T=64, H=256, I=128, E=4, topk=1), None, PRE),
    # 64 and 48 groups per row: the scale/bias staging runs in two segments
    "pre_g32_two_segments": (spec(T=48, H=2048, I=1536, E=3, topk=2, bits13=4, group13=32,
                                  bits2=2, group2=32, **ACT), None, PRE),
    # degenerate shapes: one expert over several 64-row tiles, and the
    # smallest hidden and intermediate sizes (128)
    "pre_single_expert_4_tiles": (spec(T=200, H=256, I=128, E=1, topk=1, **ACT), None, PRE),
    "dec_min_hidden": (spec(T=3, H=128, I=128, E=4, topk=2), None, DEC),
    "pre_min_hidden": (spec(T=70, H=128, I=128, E=2, topk=2, bits13=2, bits2=2), None, PRE),
    # the documented maximums: 1024 experts, top-64 (every expert of a token)
    "dec_max_experts": (spec(T=16, H=256, I=128, E=1024, topk=8), None, DEC),
    "dec_max_topk": (spec(T=4, H=256, I=128, E=64, topk=64, **ACT), None, DEC),
    "pre_max_experts": (spec(T=1024, H=256, I=128, E=1024, topk=8, bits13=2, bits2=2),
                        None, PRE),
    "pre_max_topk": (spec(T=40, H=256, I=128, E=64, topk=64, group13=64, group2=32),
                     None, PRE),
    # the largest sizes the decode-shaped kernels take (their LDS image at
    # the 64 KB limit: 5376 for groups of 128, 3328 for 2-bit groups of 32),
    # one step past it (the tile kernel), the largest single-launch hidden
    # size, and a long K for the tile kernel (128 chunks, 32 w2 column blocks)
    "dec_lds_limit_h5376": (spec(T=4, H=5376, I=256, E=8, topk=2, bits13=2, bits2=2, **ACT),
                            None, DEC),
    "pre_past_lds_limit_h5504": (spec(T=4, H=5504, I=256, E=8, topk=2, bits13=2, bits2=2),
                                 None, PRE),
    "dec_lds_limit_i5376": (spec(T=4, H=256, I=5376, E=8, topk=2, **ACT), None, DEC),
    "dec_lds_limit_g32_h3328": (spec(T=4, H=3328, I=256, E=8, topk=2, bits13=2, group13=32,
                                     bits2=2, group2=32), None, DEC),
    "dec_single_launch_h5120": (spec(T=4, H=5120, I=512, E=8, topk=2, **ACT), None, DEC),
    "pre_h16384": (spec(T=6, H=16384, I=256, E=4, topk=2, **ACT), None, PRE),
    # H = 640: the last w2 column block is partly idle (640 = 512 + 128)
    "pre_w2_partial_column_block": (spec(T=64, H=640, I=384, E=3, topk=2, bits13=2,
                                         group13=64, bits2=4, group2=128), None, PRE),
}


def forced_ids(kind, sp):
    T, k, E = sp.T, sp.topk, sp.E
    if kind == "65each":           # 4 experts x 65 pairs: 64-row tile + 1-row tail
        flat = np.repeat(np.arange(E), T * k // E)
        return np.random.default_rng(0).permutation(flat).reshape(T, k).astype(np.int32)
    if kind == "345":              # experts 0/1/2 get 5/4/3 pairs, 3 empty, rest spread
        flat = np.concatenate([np.full(5, 0), np.full(4, 1), np.full(3, 2),
                               np.arange(T * k - 12) % 4 + 4])
        return np.random.default_rng(2).permutation(flat).reshape(T, k).astype(np.int32)
    if kind == "151617":           # experts 0/1/2 get 17/16/15 pairs, 3 empty, rest spread
        flat = np.concatenate([np.full(17, 0), np.full(16, 1), np.full(15, 2),
                               np.arange(T * k - 48) % 4 + 4])
        ids = np.random.default_rng(1).permutation(flat).reshape(T, k)
        # keep ids distinct per token where possible
        return ids.astype(np.int32)
    raise ValueError(kind)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_matches_oracle(dev, name):
    sp, forced, variant = SMALL[name]
    L = make_layer(sp, seed=zlib.crc32(name.encode()) % 1000)
    if forced:
        L.topk_ids = forced_ids(forced, sp)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    assert plan["w13_variant"] == variant and plan["w2_variant"] == variant
    _, got = G.run_layer(L, dev)
    ref = O.forward_layer(L)
    G.assert_parity(got, ref, name)


@pytest.mark.parametrize("HI", [256, 1024])   # decode GEMMs in separate / shared launches
def test_layer_empty_experts_invalid_and_duplicate_ids(dev, HI):
    sp = spec(T=10, H=HI, I=HI, topk=3, E=8)
    L = make_layer(sp, seed=77)
    ids = L.topk_ids.copy()
    ids[0, 1] = -1
    ids[1, 2] = 8          # == E: out of range
    ids[2, 0] = 1000
    ids[3, 1] = ids[3, 0]  # duplicate within a token
    ids[ids == 5] = 6      # expert 5 empty
    L.topk_ids = ids.astype(np.int32)
    _, got = G.run_layer(L, dev)
    G.assert_parity(got, O.forward_layer(L), "edge ids")


@pytest.mark.parametrize("T,E", [(6, 8), (64, 4)])   # decode-shaped, prefill-shaped
def test_token_without_valid_ids_gets_zero_output(dev, T, E):
    sp = spec(T=T, topk=2, E=E)
    L = make_layer(sp, seed=78)
    L.topk_ids[1, :] = [-1, E]           # token 1: no valid id
    L.topk_ids[3, 0] = -5                # token 3: one valid id left
    y, got = G.run_layer(L, dev)
    G.assert_parity(got, O.forward_layer(L), "no valid ids")
    assert not G.to_f64(y)[1].any()


@pytest.mark.parametrize("T,E,HI", [(4, 8, 256), (4, 8, 1024), (64, 4, 256)])
def test_all_ids_invalid_overwrites_output_with_zeros(dev, T, E, HI):
    """No tile at all: the output buffer (pre-filled with garbage) must still
    be written, as the rounding of the zeroed sum (decode shapes with separate
    and with shared GEMM launches, and prefill shapes)."""
    sp = spec(T=T, H=HI, I=HI, topk=2, E=E)
    L = make_layer(sp, seed=79)
    L.topk_ids[:, :] = -1
    L.topk_ids[0, 1] = E
    out = torch.full((sp.T, sp.H), 3.0, dtype=torch.bfloat16, device=dev)
    y, got = G.run_layer(L, dev, out=out)
    assert not G.to_f64(y).any()
    G.assert_parity(got, O.forward_layer(L), "all ids invalid")


@pytest.mark.parametrize("T,E,HI,q", [(4, 8, 1024, (2, 128)), (4, 8, 1024, (4, 64)),
                                      (4, 8, 256, (4, 128)), (64, 4, 256, (4, 128))])
def test_profiled_entry_matches_plain_and_records_events(dev, T, E, HI, q):
    """The profiled entry launches the same kernels: same parity, and every
    event pair brackets a non-negative interval, launches in stream order."""
    import ctypes

    from bench import Hip

    sp = spec(T=T, H=HI, I=HI, topk=2, E=E, bits13=q[0], group13=q[1], bits2=q[0], group2=q[1])
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, q, q)
    assert plan["gemms_one_launch"] == (1 if HI == 1024 else 0)
    L = make_layer(sp, seed=80)
    d = G.to_device(L, dev)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    out = torch.empty((sp.T, sp.H), dtype=torch.bfloat16, device=dev)
    hip = Hip()
    ev = (ctypes.c_void_p * 8)(*[hip.event() for _ in range(8)])
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    clamp = None if math.isinf(sp.clamp) else sp.clamp
    st = M.moe_wna16_forward_profiled(
        d["x"].data_ptr(), d["topk_ids"].data_ptr(), d["topk_w"].data_ptr(), d["w13"].data_ptr(),
        d["s13"].data_ptr(), d["w2"].data_ptr(), d["s2"].data_ptr(), sp.T, sp.H, sp.I, sp.E,
        sp.topk, (sp.bits13, sp.group13), (sp.bits2, sp.group2), sp.alpha, sp.beta, sp.clamp,
        out.data_ptr(), ws.data_ptr(), ws.numel(), stream, ev)
    assert st == 0
    torch.cuda.synchronize(dev)
    f32 = M.workspace_f32_sum(ws, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits, G.f32_to_bf16_bits(f32))
    G.assert_parity(f32.astype(np.float64), O.forward_layer(L), "profiled entry")
    # launches in stream order: (start, stop) event indices of each launch
    launches = [(0, 1)] + ([(2, 5)] if plan["gemms_one_launch"] else [(2, 3), (4, 5)])
    if not plan["convert_in_w2"]:
        launches.append((6, 7))
    if plan["single_launch"]:
        launches = [(0, 5)]
    for a0, a1 in launches:
        assert hip.elapsed_ms(ev[a0], ev[a1]) >= 0.0
    for (_, a1), (b0, _) in zip(launches, launches[1:]):
        assert hip.elapsed_ms(ev[a1], ev[b0]) >= 0.0
    for e in ev:
        hip.destroy(e)


def test_layer_empty_batch(dev):
    L = make_layer(spec(T=0), seed=1)
    y, _ = G.run_layer(L, dev)
    assert tuple(y.shape) == (0, 256)


def test_swapped_gate_up_halves_would_fail(dev):
    """The fused w13 keeps gate rows first; an oracle fed the halves swapped
    must disagree with the library by more than the tolerance."""
    sp = spec(T=16, H=256, I=128, topk=2, **ACT)
    L = make_layer(sp, seed=9)
    _, got = G.run_layer(L, dev)
    G.assert_parity(got, O.forward_layer(L), "true layout")
    I = sp.I
    Ls = make_layer(sp, seed=9)
    Ls.w13 = np.concatenate([L.w13[:, I:], L.w13[:, :I]], axis=1).copy()
    Ls.s13 = np.concatenate([L.s13[:, I:], L.s13[:, :I]], axis=1).copy()
    assert G.parity_ratio(got, O.forward_layer(Ls)) > 1.0


def test_repeat_runs_stay_within_tolerance(dev):
    sp = spec(T=64, H=512, I=256, E=8, topk=4)
    L = make_layer(sp, seed=3)
    d = G.to_device(L, dev)
    ref = O.forward_layer(L)
    outs = [G.run_layer(L, dev, d)[1] for _ in range(4)]
    for y in outs:
        G.assert_parity(y, ref, "repeat")


def test_reused_workspace_and_output(dev):
    """A second call with a smaller batch on the same workspace and output
    buffers is unaffected by the first."""
    big = make_layer(spec(T=48, topk=2), seed=11)
    small = make_layer(spec(T=6, topk=2), seed=12)
    ws = M.workspace_for(48, 256, 128, 8, 2, dev)
    out = torch.empty((48, 256), dtype=torch.bfloat16, device=dev)
    G.run_layer(big, dev, workspace=ws, out=out)
    _, y = G.run_layer(small, dev, workspace=ws, out=out[:6])
    G.assert_parity(y, O.forward_layer(small), "reuse")


@pytest.mark.parametrize("case", ["one_token_top64", "one_expert", "two_experts_ragged"])
def test_single_launch_edge_routings(dev, case):
    """Single-launch edge cases at the 64-pair limit: one token with top-64
    over 64 experts (every tile one pair plus padding), 64 pairs on one
    expert (16 full tiles of one expert), and two experts with 61 + 3 pairs
    (ragged last tiles)."""
    if case == "one_token_top64":
        sp = spec(T=1, H=1024, I=1024, E=64, topk=64, bits13=2, bits2=2, **ACT)
    else:
        sp = spec(T=16, H=1024, I=1024, E=16, topk=4, bits13=2, bits2=2, **ACT)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (2, 128), (2, 128))
    assert plan["single_launch"] == 1
    L = make_layer(sp, seed=140)
    if case == "one_expert":
        L.topk_ids[:, :] = 5          # duplicates within every token
    elif case == "two_experts_ragged":
        ids = np.full(sp.T * sp.topk, 2, np.int32)
        ids[[7, 30, 63]] = 6
        L.topk_ids = ids.reshape(sp.T, sp.topk)
    _, got = G.run_layer(L, dev)
    G.assert_parity(got, O.forward_layer(L), case)


@pytest.mark.parametrize("q", [(2, 64), (2, 128), (4, 32), (4, 64), (4, 128)])
def test_single_launch_back_to_back_calls(dev, q):
    """The single-launch decode plan (routing, reorder, zeroing, both GEMMs
    and the rounding in one launch, ordered by counters in the workspace):
    four calls enqueued back to back on one workspace, without a host sync
    in between, with plain, duplicate, partly invalid and all-invalid ids;
    each call's output (kept in its own buffer) matches the oracle, and the
    counters are back at zero afterwards."""
    sp = spec(T=8, H=1024, I=1024, E=16, topk=8, bits13=q[0], group13=q[1], bits2=q[0],
              group2=q[1], **ACT)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, q, q)
    assert plan["single_launch"] == 1   # 64 pairs: the largest single-launch batch
    layers = []
    for seed, kind in ((90, "plain"), (91, "dup"), (92, "bad"), (93, "allbad")):
        L = make_layer(sp, seed=seed)
        if kind == "dup":
            L.topk_ids[:, 1] = L.topk_ids[:, 0]
            L.topk_ids[2, :] = L.topk_ids[2, 0]   # one expert holds all of token 2's slots
        elif kind == "bad":
            L.topk_ids[1, :] = -1
            L.topk_ids[5, 3] = sp.E
        elif kind == "allbad":
            L.topk_ids[:, :] = sp.E + 1
        layers.append(L)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    outs = []
    for L in layers:
        d = G.to_device(L, dev)
        outs.append(M.forward(d["x"], d["topk_ids"], d["topk_w"], d["w13"], d["s13"], d["w2"],
                              d["s2"], bits=(q[0], q[0]), group=(q[1], q[1]), alpha=sp.alpha,
                              beta=sp.beta, clamp=sp.clamp, workspace=ws))
    torch.cuda.synchronize(dev)
    meta = M.workspace_meta(ws, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()
    assert meta[2] == 0
    G.assert_sync_clear(ws, sp)
    G.assert_layer_sort(layers[-1], ws)
    for L, y in zip(layers, outs):
        G.assert_parity(G.to_f64(y), O.forward_layer(L), "single launch")
    assert not G.to_f64(outs[-1]).any()


@pytest.mark.parametrize("T", [8, 40])
@pytest.mark.parametrize("prepared", [False, True])
def test_decode_w2g128_i2048(dev, T, prepared):
    """2-bit group-128 decode at I = 2048 (the decode workloads' format and
    intermediate size), checkpoint and prepared codes, in the single launch
    (16 pairs) and in the shared w13 + w2 launch (80 pairs)."""
    sp = spec(T=T, H=1024, I=2048, E=32, topk=2, bits13=2, bits2=2, scale_lo=0.01,
              scale_hi=0.05, **ACT)
    q = (2, 128)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, q, q)
    assert plan["gemms_one_launch"] == 1
    assert plan["single_launch"] == (1 if T * 2 <= 64 else 0)
    L = make_layer(sp, seed=95 + T)
    _, got = G.run_layer(L, dev, prepared=prepared)
    G.assert_parity(got, O.forward_layer(L), "2-bit g128, I=2048")


@pytest.mark.parametrize("q,H,ksplit", [((2, 128), 4096, 4), ((2, 64), 4096, 4),
                                        ((4, 32), 2048, 4), ((4, 64), 4096, 4),
                                        ((4, 128), 4096, 4), ((2, 128), 2048, 2)])
def test_single_launch_split_gate_up(dev, q, H, ksplit):
    """Few tiles in the single launch (I = 512, one GPU's share under tensor
    parallelism 4): each gate/up (tile, column block) runs as `ksplit` K-slice
    workgroups whose partial sums the last one completes; plain, partly
    invalid ids, and prepared codes, on one workspace (run_layer also checks
    the counters are clear after each call)."""
    sp = spec(T=4, H=H, I=512, E=64, topk=6, bits13=q[0], group13=q[1], bits2=q[0],
              group2=q[1], **ACT)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, q, q)
    assert plan["single_launch"] == 1 and plan["w13_ksplit"] == ksplit
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    for seed, kind, prepared in ((120, "plain", False), (121, "bad", False),
                                 (122, "plain", True)):
        L = make_layer(sp, seed=seed)
        if kind == "bad":
            L.topk_ids[1, :3] = -1
            L.topk_ids[2, 0] = sp.E
        _, got = G.run_layer(L, dev, workspace=ws, prepared=prepared)
        G.assert_parity(got, O.forward_layer(L), f"split gate/up, {kind}")


@pytest.mark.parametrize("q", [(2, 128), (4, 128), (4, 64)])
def test_shared_launch_small_intermediate(dev, q):
    """96 pairs at I = 512: the shared w13 + w2 launch (not the single one)
    with the w2 prefetch depth that I allows (half the usual for 2- and
    4-bit group-128 codes), checkpoint and prepared codes."""
    sp = spec(T=16, H=1024, I=512, E=32, topk=6, bits13=q[0], group13=q[1], bits2=q[0],
              group2=q[1], **ACT)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, q, q)
    assert plan["gemms_one_launch"] == 1 and plan["single_launch"] == 0
    for prepared in (False, True):
        L = make_layer(sp, seed=130 + int(prepared))
        _, got = G.run_layer(L, dev, prepared=prepared)
        G.assert_parity(got, O.forward_layer(L), "shared launch, I = 512")


# --------------------------------------------------------------------------
# full-size workloads, sampled tokens
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_workload_sampled_tokens(dev, cfg):
    """The workloads at full size, in the launch configuration bench.py times:
    every token of the decode workloads, and 64 tokens of each prefill
    workload chosen at the XCD range boundaries, the first and last tile and
    the least-used experts.  The layer's own sort is checked bit for bit
    (run_layer)."""
    L = make_config(cfg)
    sp = L.spec
    print(f"config {cfg} {sp.name}: T={sp.T} E={sp.E} k={sp.topk}", flush=True)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    _, y = G.run_layer(L, dev, workspace=ws)
    assert np.all(np.isfinite(y))
    rows = list(range(sp.T)) if sp.T <= 64 else G.sampled_tokens(L, ws)
    assert len(rows) == min(sp.T, 64)
    ref = O.forward_layer(L, tokens=rows)
    G.assert_parity(y[rows], ref, f"config {cfg}")
    if cfg in (4, 5):   # 372 and 1139 tiles: the split's chunk carry (above 1024)
        G.assert_xcd_split(L, ws)


@pytest.mark.parametrize("shard", ["ep8", "tp4"])
@pytest.mark.parametrize("cfg", [2, 4])
def test_one_gpu_share_of_sharded_layer(dev, cfg, shard):
    """One GPU's share of the sharded layer at its real shape: expert
    parallelism over 8 GPUs (32 local experts receiving the global top-k ids
    over 256 experts; the other ids contribute nothing here) and tensor
    parallelism over 4 (intermediate 512), for the decode and the 2048-token
    prefill workloads.  The partial sums of the shares are what the
    cross-GPU reduction would add."""
    sp = shard_spec(cfg, shard)
    L = make_layer(sp, seed=cfg)
    print(f"{sp.name}: T={sp.T} E={sp.E} I={sp.I} k={sp.topk}", flush=True)
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    _, y = G.run_layer(L, dev, workspace=ws)
    rows = list(range(sp.T)) if sp.T <= 64 else G.sampled_tokens(L, ws)
    G.assert_parity(y[rows], O.forward_layer(L, tokens=rows), sp.name)
    if shard == "ep8":
        local = (L.topk_ids >= 0) & (L.topk_ids < sp.E)
        assert G.layer_sort(L, ws)[1]["bad_ids"] == int((~local).sum())


@pytest.mark.parametrize("T,k,routing,bad", [(896, 8, "zipf", False), (7169, 1, "uniform", True),
                                             (2048, 4, "zipf", False), (2048, 6, "zipf", True),
                                             (8192, 8, "zipf", True)])
def test_layer_sort_bit_exact_across_sort_paths(dev, T, k, routing, bad):
    """The layer's own expert sort on both sides of the route kernel's switch
    from recounting every pair (up to 7 sort workgroups: P = 7168) to summing
    per-chunk counts from the count launch (8 and more: P = 7169, 8192,
    12288, 65536), 64-row tiles, 256 experts: sorted ids, tile experts,
    offsets, inverse permutation and tile count equal the oracle's bit for
    bit (run_layer), with invalid ids counted in some cases, and the layer
    output within tolerance."""
    P = T * k
    sp = spec(T=T, H=128, I=128, E=256, topk=k, routing=routing, bits13=2, bits2=2, **ACT)
    L = make_layer(sp, seed=P)
    if bad:
        flat = L.topk_ids.reshape(-1).copy()
        where = np.random.default_rng(P).choice(P, size=15, replace=False)
        flat[where] = np.repeat([-1, 256, 1 << 20], 5)
        L.topk_ids = flat.reshape(T, k)
    plan = M.moe_wna16_plan(T, 128, 128, 256, k, (2, 128), (2, 128))
    assert plan["block_m"] == 64
    # sort workgroups: chunks of a multiple of 1024 pairs, at most 16 of them
    per = math.ceil(P / 16)
    chunk = max(1024, math.ceil(per / 1024) * 1024)
    assert (math.ceil(P / chunk) >= 8) == (P >= 7169)
    ws = M.workspace_for(T, 128, 128, 256, k, dev)
    _, got = G.run_layer(L, dev, workspace=ws)
    assert G.layer_sort(L, ws)[1]["bad_ids"] == (15 if bad else 0)
    G.assert_parity(got, O.forward_layer(L), f"P={P}")


def test_tile_split_beyond_4096_tiles(dev):
    """5120 tiles of 64 rows (1024 experts with 257 pairs each): the XCD split
    recomputes the costs of tiles past its register cache (4096 tiles) and
    carries its scan over five 1024-tile chunks.  Its ranges must equal the
    host model, and every token's output the oracle's."""
    E, k = 1024, 8
    T = 257 * E // k
    sp = spec(T=T, H=128, I=128, E=E, topk=k, **ACT)
    L = make_layer(sp, seed=33)
    L.topk_ids = (np.arange(T * k, dtype=np.int64).reshape(T, k) % E).astype(np.int32)
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    assert plan["w13_variant"] == PRE and plan["block_m"] == 64
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    _, got = G.run_layer(L, dev, workspace=ws)
    assert int(G.workspace_meta(ws, sp)[0]) == 5 * E
    G.assert_xcd_split(L, ws)
    G.assert_parity(got, O.forward_layer(L), "5120 tiles")


def test_tile_split_ranges_capped_at_launch_slots(dev):
    """Prefill-shaped plan whose cost-balanced XCD split needs the cap: 108
    full 64-row tiles of expert 0 followed by 27 one-row experts.  With one
    column block per GEMM each XCD gets 26 workgroup slots, and the balanced
    split would give the last XCD the 27 one-row tiles.  The capped ranges must
    still cover every item once (checked through the output), and the table
    the split kernel leaves in the workspace (ints 8..25: w13 then w2, 8 range
    starts and the total each) must respect the cap."""
    nfull, nsmall = 108, 27
    T = 64 * nfull + nsmall
    sp = spec(T=T, H=512, I=256, E=nsmall + 1, topk=1, **ACT)
    L = make_layer(sp, seed=31)
    ids = np.zeros((T, 1), np.int32)
    ids[64 * nfull:, 0] = np.arange(1, nsmall + 1)
    L.topk_ids = ids
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    assert plan["w13_variant"] == PRE and plan["block_m"] == 64
    ws = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    _, got = G.run_layer(L, dev, workspace=ws)
    G.assert_parity(got, O.forward_layer(L), "capped XCD split")
    G.assert_xcd_split(L, ws)
    table = ws[:128].view(torch.int32)[8:26].cpu().numpy().reshape(2, 9)
    ntiles = nfull + nsmall
    max_tiles = plan["max_tiles"]
    per = (max_tiles + 7) // 8
    cap = per + per // 2 + 1          # slots per XCD with one column block
    for first in table:
        lens = np.diff(first)
        assert first[0] == 0 and first[8] == ntiles, first
        assert np.all(lens >= 0) and np.all(lens <= cap), (first, cap)
        assert lens.max() == cap, (first, cap)   # the cap did bind
