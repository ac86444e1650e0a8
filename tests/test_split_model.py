"""Host model of the tile kernels' XCD split (tests/_gpu.py), on cases worked
out by hand; the GPU tests compare the split the layer ran against it."""
from tests import _gpu as G


def ids_for(rows_per_tile, P):
    """sorted_ids of 64-row tiles with the given real rows (padding = P)."""
    out = []
    for n in rows_per_tile:
        out += list(range(n)) + [P] * (64 - n)
    return out


def test_equal_tiles_split_evenly():
    # 8 full tiles, cost 7 each, one column block: one tile per XCD
    B = G.xcd_split_model(ids_for([64] * 8, 10 ** 6), 8, 10 ** 6, nblk=1, cap=100)
    assert B == [0, 1, 2, 3, 4, 5, 6, 7, 8]


def test_split_inside_a_tile_by_cost():
    # 2 tiles (costs 7 and 4), 4 column blocks each; C = 11: range x starts at
    # cost x * 11 / 8, so x = 1..5 fall in tile 0 (cost 7 of 11 -> items
    # ceil(4 * x*11 / (8*7))), x = 6, 7 in tile 1
    B = G.xcd_split_model(ids_for([64, 1], 10 ** 6), 2, 10 ** 6, nblk=4, cap=100)
    want = [0]
    for x in range(1, 8):
        t = 11 * x
        if t <= 8 * 7:
            want.append(-(-4 * t // 56))
        else:
            want.append(4 + -(-4 * (t - 56) // 32))
    assert B == want + [8]
    assert B == [0, 1, 2, 3, 4, 4, 6, 7, 8]


def test_cap_limits_every_range():
    # all cost in the first tile; a cap of 3 items per XCD pushes the starts
    # forward and back so that no range exceeds 3 and all 16 items stay covered
    B = G.xcd_split_model(ids_for([64] + [1] * 3, 10 ** 6), 4, 10 ** 6, nblk=4, cap=3)
    lens = [b - a for a, b in zip(B, B[1:])]
    assert B[0] == 0 and B[8] == 16
    assert all(0 <= n <= 3 for n in lens), B
    assert sorted(B) == B


def test_no_tiles():
    assert G.xcd_split_model([], 0, 5, nblk=2, cap=3) == [0] * 9
