"""The random-shape parity cases (tests/_random_shapes.py) reach every path
of the plan and stay within the oracle's budget."""
import weight_only_bit_moe_amd as M
from tests._random_shapes import MAX_MACS, SEEDS, random_spec


def _plans():
    out = []
    for seed in SEEDS:
        sp = random_spec(seed)
        out.append((sp, M.moe_wna16_plan(sp.T, sp.H, sp.I, sp.E, sp.topk,
                                         (sp.bits13, sp.group13), (sp.bits2, sp.group2))))
    return out


def test_random_shapes_cover_every_path():
    plans = _plans()
    assert any(p["w13_variant"] == 1 for _, p in plans)
    assert any(p["w13_variant"] == 2 and p["gemms_one_launch"] == 0 for _, p in plans)
    assert any(p["gemms_one_launch"] == 1 and p["single_launch"] == 0 for _, p in plans)
    assert sum(p["single_launch"] for _, p in plans) >= 3
    assert {sp.bits13 for sp, _ in plans} == {2, 4} and {sp.bits2 for sp, _ in plans} == {2, 4}
    assert {sp.group13 for sp, _ in plans} == {32, 64, 128}
    assert {sp.group2 for sp, _ in plans} == {32, 64, 128}


def test_random_shapes_fit_the_oracle_budget():
    for sp, _ in _plans():
        assert 3.0 * sp.T * sp.topk * sp.H * sp.I <= MAX_MACS, sp
