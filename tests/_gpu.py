"""Helpers shared by the GPU tests: move a synthetic layer to the device, run
the HIP library through its C ABI, and compare with the oracle.

The layer's result is an FP32 sum rounded once to BF16.  Parity is checked on
the FP32 sum (read back from the workspace) against the oracle with the
stated bound, and the BF16 output must equal the round-to-nearest-even of
that sum bit for bit.  (Rounding the exact result to BF16 can by itself
exceed 2e-2 * rms when the output has heavy tails, so the bound cannot be
applied after the rounding.)"""
import math

import numpy as np
import torch

import weight_only_bit_moe_amd as M
from weight_only_bit_moe_amd.inputs import f32_to_bf16_bits

#: Elementwise bound for the layer output: |gpu - oracle| <= REL * rms(oracle) + ABS,
#: with rms over every output element compared.
REL, ABS = 2e-2, 1e-3


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_device(L, dev):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(
        x=torch.from_numpy(L.x.view(np.int16)).to(dev).view(torch.bfloat16),
        topk_ids=t(L.topk_ids, np.int32),
        topk_w=t(L.topk_w, np.float32),
        w13=torch.from_numpy(L.w13.view(np.int32)).to(dev),
        s13=torch.from_numpy(L.s13).to(dev),
        w2=torch.from_numpy(L.w2.view(np.int32)).to(dev),
        s2=torch.from_numpy(L.s2).to(dev),
    )


def run_layer(L, dev, d=None, out=None, workspace=None, prepared=False, check_sort=True):
    """Run the layer; returns (BF16 output tensor, FP32 sum as float64 numpy).
    Also checks that the output is the RNE rounding of the FP32 sum, that no
    fused decode wait gave up, and (check_sort) that the expert sort the
    layer itself ran -- read back from its workspace -- equals the oracle's
    bit for bit at the plan's tile size.  With prepared=True the codes are
    first put in the prepared order on the GPU and the prepared entry point
    runs."""
    sp = L.spec
    d = d or to_device(L, dev)
    clamp = None if math.isinf(sp.clamp) else sp.clamp
    if workspace is None:
        workspace = M.workspace_for(sp.T, sp.H, sp.I, sp.E, sp.topk, dev)
    w13, w2 = d["w13"], d["w2"]
    if prepared:
        w13 = M.prepare(w13, sp.bits13, sp.group13)
        w2 = M.prepare(w2, sp.bits2, sp.group2)
    y = M.forward(d["x"], d["topk_ids"], d["topk_w"], w13, d["s13"], w2, d["s2"],
                  bits=(sp.bits13, sp.bits2), group=(sp.group13, sp.group2), alpha=sp.alpha,
                  beta=sp.beta, clamp=clamp, out=out, workspace=workspace, prepared=prepared)
    torch.cuda.synchronize(dev)
    if sp.T == 0:
        return y, np.zeros((0, sp.H))
    f32 = M.workspace_f32_sum(workspace, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()
    bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits, f32_to_bf16_bits(f32)), "BF16 output is not RNE(FP32 sum)"
    meta = M.workspace_meta(workspace, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()
    assert meta[2] == 0, f"{meta[2]} fused decode waits gave up"
    assert_sync_clear(workspace, sp)
    if check_sort:
        assert_layer_sort(L, workspace)
    return y, f32.astype(np.float64)


def assert_sync_clear(workspace, sp):
    """The single-launch decode's counters (workspace bytes [256,
    SYNC_BYTES) past the status words) are back at zero after a call."""
    at = M.moe_wna16_workspace_layout(sp.T, sp.H, sp.I, sp.E, sp.topk)["meta"]
    sync = workspace[at + 256:at + M.SYNC_BYTES].cpu().numpy()
    assert not sync.any(), f"sync counters left non-zero at bytes {np.flatnonzero(sync)[:8]}"


def xcd_split_model(sorted_ids, ntiles, P, nblk, cap):
    """Host model of the tile kernels' XCD split (the range starts the split
    launch leaves in workspace ints 8..25 for one GEMM): each tile costs 3 +
    its active 16-row slices; range x (1..7) starts at the first item whose
    preceding cost reaches x/8 of the total, inside its tile in proportion to
    the cost; the starts are kept in order, then every range is capped at
    `cap` items, forward and back."""
    cost = [3 + sum(1 for s in range(4) if sorted_ids[b * 64 + 16 * s] < P)
            for b in range(ntiles)]
    C = sum(cost)
    B = [0] * 9
    B[8] = ntiles * nblk
    S = 0
    for b, c in enumerate(cost):
        for x in range(1, 8):
            t = x * C
            if 8 * S < t <= 8 * (S + c):
                num, den = t - 8 * S, 8 * c
                B[x] = b * nblk + (nblk * num + den - 1) // den
        S += c
    for x in range(1, 8):
        B[x] = max(B[x - 1], min(B[x], B[8]))
    for x in range(1, 8):
        B[x] = min(B[x], B[x - 1] + cap)
    for x in range(7, 0, -1):
        B[x] = max(B[x], B[x + 1] - cap)
    return B


def xcd_split_caps(plan, H, I):
    """(nblk, cap) of the w13 and w2 tile launches: 256 gate/up output
    columns and 512 down output columns per workgroup; slots per XCD = 1.5 x
    the even share of max_tiles items plus one tile's items."""
    out = []
    for n, outc in ((I, 256), (H, 512)):
        nblk = -(-n // outc)
        per = -(-plan["max_tiles"] * nblk // 8)
        out.append((nblk, per + per // 2 + nblk))
    return out


def assert_xcd_split(L, workspace):
    """The split the layer ran (workspace ints 8..25) equals the host model."""
    sp = L.spec
    plan = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                            (sp.bits2, sp.group2))
    assert plan["block_m"] == 64
    srt = M.workspace_sort(workspace, sp.T, sp.H, sp.I, sp.E, sp.topk, 64)
    ntiles = int(srt["num_tiles"])
    sorted_ids = srt["sorted_ids"]
    table = workspace_meta(workspace, sp)[8:26].reshape(2, 9)
    for got, (nblk, cap) in zip(table, xcd_split_caps(plan, sp.H, sp.I)):
        want = xcd_split_model(sorted_ids, ntiles, sp.T * sp.topk, nblk, cap)
        assert list(got) == want, (list(got), want)


def workspace_meta(workspace, sp):
    return M.workspace_meta(workspace, sp.T, sp.H, sp.I, sp.E, sp.topk).cpu().numpy()


def layer_sort(L, workspace):
    """The expert sort a completed forward on layer L ran (plan's block_m)."""
    sp = L.spec
    bm = M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk, (sp.bits13, sp.group13),
                          (sp.bits2, sp.group2))["block_m"]
    return bm, M.workspace_sort(workspace, sp.T, sp.H, sp.I, sp.E, sp.topk, bm)


def assert_align_equal(got, ref):
    assert got["num_tiles"] == ref["num_tiles"], (got["num_tiles"], ref["num_tiles"])
    assert got["bad_ids"] == ref["bad_ids"], (got["bad_ids"], ref["bad_ids"])
    for k in ("sorted_ids", "tile_expert", "expert_offsets", "inv_perm"):
        assert np.array_equal(got[k], ref[k]), k


def assert_layer_sort(L, workspace):
    """The layer's own sort equals the oracle's, bit for bit."""
    from oracle import oracle as O
    bm, got = layer_sort(L, workspace)
    assert_align_equal(got, O.align(L.topk_ids, L.spec.E, bm))


def to_f64(y):
    return y.float().cpu().numpy().astype(np.float64)


def parity_ratio(got, ref):
    """max |got - ref| / (REL * rms(ref) + ABS) over all compared elements."""
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    tol = REL * rms + ABS
    return float(np.max(np.abs(got - ref))) / tol if ref.size else 0.0


def assert_parity(got, ref, what=""):
    r = parity_ratio(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r <= 1.0, f"{what}: max error is {r:.3f}x the tolerance"
    return r


def sampled_tokens(L, ws, n=64):
    """Tokens of a full-size prefill-shaped layer worth checking one by one:
    those in the tiles on both sides of every XCD range boundary of both
    GEMMs (read from the split table the layer left in its workspace), the
    first and last tile, tokens routed to the 8 least-used experts, then
    evenly spaced tokens up to n."""
    sp = L.spec
    T, k = sp.T, sp.topk
    bm, srt = layer_sort(L, ws)
    meta = M.workspace_meta(ws, T, sp.H, sp.I, sp.E, k).cpu().numpy()
    ntiles = srt["num_tiles"]
    picked = []

    def add_tile(b):
        if 0 <= b < ntiles:
            rows = srt["sorted_ids"][b * bm:(b + 1) * bm]
            real = rows[rows < T * k]
            picked.extend([int(real[0]) // k, int(real[-1]) // k])

    if bm == 64:
        for g, outc, N in ((0, 256, sp.I), (1, 512, sp.H)):   # items per tile: column blocks
            nblk = -(-N // outc)
            first = meta[8 + 9 * g: 17 + 9 * g]
            for x in range(1, 8):
                add_tile(int(first[x]) // nblk)
                add_tile((int(first[x]) - 1) // nblk)
    add_tile(0)
    add_tile(ntiles - 1)
    ids = L.topk_ids
    counts = np.bincount(ids[(ids >= 0) & (ids < sp.E)].ravel(), minlength=sp.E)
    for e in np.argsort(np.where(counts > 0, counts, 1 << 30), kind="stable")[:8]:
        if counts[e]:
            picked.append(int(np.argwhere(ids == e)[0][0]))
    out = list(dict.fromkeys(picked))[:n]
    for t in np.linspace(0, T - 1, n).astype(int):
        if len(out) >= n:
            break
        if t not in out:
            out.append(int(t))
    return sorted(out)
