"""The C-ABI library: it loads, exports every function include/moe_wna16.h
declares, and rejects bad arguments on the host before any device call."""
import ctypes
import math
import os
import re

import pytest

import weight_only_bit_moe_amd as M
from weight_only_bit_moe_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_wna16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_wna16_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        pytest.fail(f"{M.LIB_PATH} not built (python -m weight_only_bit_moe_amd.build)")
    return M.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names == sorted(M.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert M.moe_wna16_status_string(st) not in ("", "unknown status")
    assert M.moe_wna16_status_string(99) == "unknown status"


def test_workspace_size_monotone(lib):
    a = M.moe_wna16_workspace_size(4, 4096, 2048, 256, 6)
    b = M.moe_wna16_workspace_size(64, 4096, 2048, 256, 6)
    c = M.moe_wna16_workspace_size(8192, 4096, 2048, 256, 8)
    assert 0 < a < b < c
    assert M.moe_wna16_workspace_size(0, 256, 128, 8, 2) > 0
    with pytest.raises(M.MoeWna16Error):
        M.moe_wna16_workspace_size(4, 100, 2048, 256, 6)


def test_plan_picks_tiles_from_rows_per_expert(lib):
    dec = M.moe_wna16_plan(4, 4096, 2048, 256, 6, (2, 128), (2, 128))
    bdec = M.moe_wna16_plan(64, 4096, 2048, 256, 6, (4, 128), (4, 128))
    pre = M.moe_wna16_plan(2048, 4096, 2048, 256, 6, (2, 128), (2, 128))
    # tile capacity: sum over used experts of ceil(count / bm) <= (P + (bm - 1) min(E, P)) / bm
    assert dec["block_m"] == 4 and dec["w13_variant"] == 2 and dec["max_tiles"] == 24
    assert bdec["block_m"] == 4 and bdec["w2_variant"] == 2
    assert pre["block_m"] == 64 and pre["w2_variant"] == 1
    assert pre["max_tiles"] == (2048 * 6 + 63 * 256) // 64
    # the decode kernel's LDS image must fit: a 32-group w13 at H=4096 goes prefill-shaped
    big = M.moe_wna16_plan(4, 4096, 2048, 256, 6, (4, 32), (2, 128))
    assert big["w13_variant"] == 1


def test_plan_decode_lds_limits(lib):
    """The decode-shaped kernels hold whole activation rows and the
    workgroup's scales in at most 64 KB of LDS: hidden (or intermediate)
    sizes up to 5376 for groups of 128 and 3328 for 2-bit groups of 32 stay
    decode-shaped, one step more goes to the tile kernel; the single launch
    (both GEMMs in one launch) stops at 5120."""
    for q, last in [((2, 128), 5376), ((4, 128), 5376), ((2, 32), 3328), ((4, 64), 4480)]:
        assert M.moe_wna16_plan(4, last, 256, 8, 2, q, q)["w13_variant"] == 2, q
        assert M.moe_wna16_plan(4, last + 128, 256, 8, 2, q, q)["w13_variant"] == 1, q
        assert M.moe_wna16_plan(4, 1024, last, 8, 2, q, q)["w2_variant"] == 2, q
        assert M.moe_wna16_plan(4, 1024, last + 128, 8, 2, q, q)["w2_variant"] == 1, q
    assert M.moe_wna16_plan(4, 5120, 512, 8, 2, (4, 128), (4, 128))["single_launch"] == 1
    assert M.moe_wna16_plan(4, 5248, 512, 8, 2, (4, 128), (4, 128))["single_launch"] == 0


def test_plan_reports_shared_launches(lib):
    dec = M.moe_wna16_plan(4, 4096, 2048, 256, 6, (2, 128), (2, 128))
    assert dec["gemms_one_launch"] == 1 and dec["convert_in_w2"] == 1
    bdec = M.moe_wna16_plan(64, 4096, 2048, 256, 6, (4, 128), (4, 128))
    assert bdec["gemms_one_launch"] == 1 and bdec["convert_in_w2"] == 1   # 64*4096 <= 2^18
    big_t = M.moe_wna16_plan(128, 4096, 2048, 256, 6, (4, 128), (4, 128))
    assert big_t["w13_variant"] == 2 and big_t["convert_in_w2"] == 0
    mixed = M.moe_wna16_plan(4, 4096, 2048, 256, 6, (4, 128), (2, 128))
    assert mixed["w13_variant"] == 2 and mixed["gemms_one_launch"] == 0
    g32 = M.moe_wna16_plan(4, 1024, 512, 256, 6, (2, 32), (2, 32))
    assert g32["w13_variant"] == 2 and g32["gemms_one_launch"] == 0
    pre = M.moe_wna16_plan(2048, 4096, 2048, 256, 6, (2, 128), (2, 128))
    assert pre["gemms_one_launch"] == 0 and pre["convert_in_w2"] == 0
    # the whole layer in one launch: both shared launches and at most 64 pairs
    assert dec["single_launch"] == 1
    assert bdec["single_launch"] == 0                        # 384 pairs
    edge = M.moe_wna16_plan(8, 4096, 2048, 256, 8, (4, 128), (4, 128))
    assert edge["single_launch"] == 1                        # exactly 64 pairs
    over = M.moe_wna16_plan(13, 4096, 2048, 256, 5, (4, 128), (4, 128))
    assert over["gemms_one_launch"] == 1 and over["single_launch"] == 0   # 65 pairs
    for p in (mixed, g32, pre, big_t):
        assert p["single_launch"] == 0
    # a small intermediate (one GPU's share under tensor parallelism 4) runs the
    # shared launches with half the w2 prefetch depth, and the single launch
    # splits each gate/up item's K in 4 (192 items would leave the GPU idle)
    tp4 = M.moe_wna16_plan(4, 4096, 512, 256, 6, (2, 128), (2, 128))
    assert tp4["gemms_one_launch"] == 1 and tp4["single_launch"] == 1
    assert tp4["w13_ksplit"] == 4
    assert dec["w13_ksplit"] == 1                            # 768 items already
    tp4_4b = M.moe_wna16_plan(4, 4096, 512, 256, 6, (4, 128), (4, 128))
    assert tp4_4b["single_launch"] == 1 and tp4_4b["w13_ksplit"] == 4
    for p in (bdec, pre, mixed):
        assert p["w13_ksplit"] == 1


NAN, INF = float("nan"), math.inf
GOOD = dict(T=4, H=256, I=128, E=8, topk=2, q13=(4, 128), q2=(4, 128), alpha=1.0, beta=0.0,
            clamp=INF)


def call(ptrs=16, ws_bytes=1 << 30, ws_ptr=4096, **over):
    a = dict(GOOD)
    a.update(over)
    p = ptrs
    return M.moe_wna16_forward(p, p, p, p, p, p, p, a["T"], a["H"], a["I"], a["E"], a["topk"],
                               a["q13"], a["q2"], a["alpha"], a["beta"], a["clamp"], p, ws_ptr,
                               ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(T=-1), Bd.EINVAL), (dict(H=0), Bd.EINVAL), (dict(E=0), Bd.EINVAL),
    (dict(topk=0), Bd.EINVAL), (dict(alpha=NAN), Bd.EINVAL), (dict(beta=INF), Bd.EINVAL),
    (dict(clamp=NAN), Bd.EINVAL), (dict(clamp=-1.0), Bd.EINVAL),
    (dict(q13=(3, 128)), Bd.EUNSUPPORTED), (dict(q2=(4, 96)), Bd.EUNSUPPORTED),
    (dict(H=200), Bd.EUNSUPPORTED), (dict(I=64), Bd.EUNSUPPORTED), (dict(E=1025), Bd.EUNSUPPORTED),
    (dict(topk=65), Bd.EUNSUPPORTED), (dict(I=128, q2=(2, 128)), None),
    (dict(T=1 << 20, H=2048, topk=1), Bd.EUNSUPPORTED),     # T*H*2 = 2^32
    (dict(T=1 << 17, H=256, I=2048, topk=8), Bd.EUNSUPPORTED),  # act slots * I * 2 > 2^32
])
def test_forward_rejects_before_device(lib, over, status):
    st = call(**over)
    if status is None:   # valid arguments reach the device check (no GPU here)
        assert st in (Bd.EHIP, Bd.EARCH, Bd.OK)
    else:
        assert st == status


def test_forward_null_misaligned_and_workspace(lib):
    assert call(ptrs=0) == Bd.EINVAL
    assert call(ptrs=18) == Bd.EALIGN
    assert call(ws_ptr=4096 + 16) == Bd.EALIGN
    assert call(ws_bytes=10) == Bd.EWORKSPACE
    need = M.moe_wna16_workspace_size(4, 256, 128, 8, 2)
    assert call(ws_bytes=need - 1) == Bd.EWORKSPACE
    assert call(ws_bytes=need) in (Bd.EHIP, Bd.EARCH, Bd.OK)


def test_empty_batch_is_ok_without_device(lib):
    assert call(T=0, ptrs=0, ws_ptr=0, ws_bytes=0) == Bd.OK


def test_align_rejects(lib):
    f = M.moe_wna16_align
    assert f(16, 4, 2, 0, 16, 16, 16, 16, 16, 16, 16, None) == Bd.EINVAL
    assert f(16, 4, 2, 8, 0, 16, 16, 16, 16, 16, 16, None) == Bd.EINVAL
    assert f(16, 4, 2, 2048, 16, 16, 16, 16, 16, 16, 16, None) == Bd.EUNSUPPORTED
    assert f(18, 4, 2, 8, 16, 16, 16, 16, 16, 16, 16, None) == Bd.EALIGN
    assert f(0, 4, 2, 8, 16, 16, 16, 16, 16, 16, 16, None) == Bd.EINVAL


def test_library_carries_gfx950_code_only(lib):
    """The shared object embeds an offload bundle for gfx950 (our own build)."""
    blob = open(M.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


def test_quantize_rejects(lib):
    f = M.moe_wna16_quantize
    ok = dict(w=256, imp=None, rows=4, K=256, q=(4, 128), n_candidates=8, codes_out=256,
              scales_out=256, err_sums_out=256, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["w"], a["imp"], a["rows"], a["K"], a["q"], a["n_candidates"],
                 a["codes_out"], a["scales_out"], a["err_sums_out"], a["stream"])

    assert call(rows=-1) == Bd.EINVAL
    assert call(K=0) == Bd.EINVAL
    assert call(n_candidates=0) == Bd.EINVAL
    assert call(n_candidates=65) == Bd.EINVAL
    assert call(q=(3, 128)) == Bd.EUNSUPPORTED
    assert call(q=(4, 96)) == Bd.EUNSUPPORTED
    assert call(K=192) == Bd.EUNSUPPORTED          # not a multiple of the group
    assert call(w=0) == Bd.EINVAL
    assert call(err_sums_out=0) == Bd.EINVAL
    assert call(w=258) == Bd.EALIGN
    assert call(w=260) == Bd.EALIGN          # weights are read 16 bytes at a time
    assert call(imp=258) == Bd.EALIGN
    assert call(err_sums_out=260) == Bd.EALIGN
    assert call(scales_out=257) == Bd.EALIGN
    # an empty matrix needs no weight, code or scale buffer
    assert call(rows=0, w=0, codes_out=0, scales_out=0) in (Bd.EHIP, Bd.EARCH, Bd.OK)


def test_plan_sends_partial_load_units_to_tile_kernel(lib):
    """The decode-shaped kernels walk K in units of 512/bits elements: a 2-bit
    projection whose K is an odd multiple of 128 gets the 64-row tile kernel."""
    ok = M.moe_wna16_plan(4, 512, 256, 8, 2, (2, 128), (2, 128))
    assert ok["w13_variant"] == 2 and ok["block_m"] == 4
    for H, I, q13, q2 in [(384, 256, (2, 128), (2, 128)), (512, 384, (4, 128), (2, 128)),
                          (640, 256, (2, 64), (4, 64))]:
        p = M.moe_wna16_plan(4, H, I, 8, 2, q13, q2)
        assert p["w13_variant"] == 1 and p["w2_variant"] == 1 and p["block_m"] == 64, (H, I)
    # 4-bit codes: units of 128 elements, so K = 384 stays decode-shaped
    p = M.moe_wna16_plan(4, 384, 384, 8, 2, (4, 128), (4, 128))
    assert p["w13_variant"] == 2


def test_prepare_rejects(lib):
    f = M.moe_wna16_prepare
    assert f(256, -1, 16, 256, (4, 128), 4096, None) == Bd.EINVAL
    assert f(256, 2, 16, 0, (4, 128), 4096, None) == Bd.EINVAL
    assert f(256, 2, 24, 256, (4, 128), 4096, None) == Bd.EUNSUPPORTED    # rows % 16
    assert f(256, 2, 16, 384, (2, 128), 4096, None) == Bd.EUNSUPPORTED    # 2-bit unit 256
    assert f(256, 2, 16, 256, (3, 128), 4096, None) == Bd.EUNSUPPORTED
    assert f(0, 2, 16, 256, (4, 128), 1 << 20, None) == Bd.EINVAL
    assert f(256, 2, 16, 256, (4, 128), 0, None) == Bd.EINVAL
    assert f(4096, 2, 16, 256, (4, 128), 4096 + 1024, None) == Bd.EINVAL  # overlap
    assert f(258, 2, 16, 256, (4, 128), 1 << 20, None) == Bd.EALIGN
    assert f(256, 2, 16, 256, (4, 128), (1 << 20) + 4, None) == Bd.EALIGN
    assert f(0, 0, 16, 256, (4, 128), 0, None) == Bd.OK                   # nothing to do


def test_forward_prepared_checks_like_forward(lib):
    """Host checks run before the layout restriction: bad sizes are EINVAL."""
    f = M.moe_wna16_forward_prepared
    args = [16] * 7 + [4, 256, 128, 8, 2, (4, 128), (4, 128), 1.0, 0.0, float("inf"), 16, 4096,
                        1 << 30, None]
    bad = list(args)
    bad[7] = -1
    assert f(*bad) == Bd.EINVAL
    assert f(*([0] * 7 + args[7:])) == Bd.EINVAL
    zero = list(args)
    zero[7] = 0
    assert f(*zero) == Bd.OK


def test_workspace_layout_consistent(lib):
    """The layout query agrees with the size and FP32-offset queries, and its
    pieces are 256-byte aligned, in bounds and large enough for their arrays."""
    for T, H, I, E, k in [(4, 4096, 2048, 256, 6), (8192, 4096, 2048, 256, 8), (0, 256, 128, 8, 2),
                          (7169, 128, 128, 256, 1)]:
        lay = M.moe_wna16_workspace_layout(T, H, I, E, k)
        assert lay["total"] == M.moe_wna16_workspace_size(T, H, I, E, k)
        assert lay["out_f32"] == M.moe_wna16_workspace_f32_offset(T, H, I, E, k)
        P = T * k
        need = {"meta": 26 * 4, "expert_offsets": (E + 1) * 4, "inv_perm": P * 4,
                "sorted_ids": (P // 4 + min(E, P)) * 4 * 4, "tile_expert": (P // 4 + min(E, P)) * 4,
                "out_f32": T * H * 4}
        spans = sorted((lay[n], lay[n] + need[n]) for n in need)
        for (a0, a1), (b0, _) in zip(spans, spans[1:]):
            assert a1 <= b0, (T, spans)
        assert spans[-1][1] <= lay["total"]
        assert all(lay[n] % 256 == 0 for n in need)
    with pytest.raises(M.MoeWna16Error):
        M.moe_wna16_workspace_layout(4, 100, 2048, 256, 6)
    assert lib.moe_wna16_workspace_layout(4, 4096, 2048, 256, 6, None) == Bd.EINVAL


def test_noalloc_rejects_oversized_calls_before_touching_the_device(lib):
    """The scratch-size check runs with the other host checks (no GPU here):
    a 2048-token prefill-shaped call needs more than 32 MiB."""
    fake = 1 << 20   # aligned, never dereferenced: the call returns first
    st = lib.moe_wna16_forward_noalloc(fake, fake, fake, fake, fake, fake, fake, 2048, 4096, 2048,
                                       256, 6, Bd.QParams(2, 128), Bd.QParams(2, 128), 1.0, 0.0,
                                       math.inf, fake, None)
    assert st == Bd.ESCRATCH
    assert "32 MiB" in M.moe_wna16_status_string(Bd.ESCRATCH)
    # bad arguments are still EINVAL / EALIGN first
    assert lib.moe_wna16_forward_noalloc(None, fake, fake, fake, fake, fake, fake, 4, 4096, 2048,
                                         256, 6, Bd.QParams(2, 128), Bd.QParams(2, 128), 1.0, 0.0,
                                         math.inf, fake, None) == Bd.EINVAL
    assert lib.moe_wna16_forward_noalloc(fake + 2, fake, fake, fake, fake, fake, fake, 4, 4096,
                                         2048, 256, 6, Bd.QParams(2, 128), Bd.QParams(2, 128),
                                         1.0, 0.0, math.inf, fake, None) == Bd.EALIGN
